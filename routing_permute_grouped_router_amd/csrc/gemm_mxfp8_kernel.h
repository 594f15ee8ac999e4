// Grouped MXFP8 GEMMs on CDNA4 scaled matrix cores
// (v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 operands, E8M0 scales per 32).
//
// Same computation and device-side group handling as the bf16 kernel
// (gemm_bf16_kernel.h), on the MXFP8 block-scaled format of the cudnn-frontend
// page "Add MoE + expert-parallel Python API surface, PyTorch reference, and
// tests" (BlockScaledTensor, block 32) with OCP E4M3 elements.
//
// These GEMMs stream their weights from HBM (each expert's weights serve only
// its own few hundred rows), so the design favours bytes in flight over
// on-chip reuse:
//   - tiles are 128 rows x 256 columns (SwiGLU: 128 gate + 128 up rows of W1),
//     so an expert with a few hundred rows wastes at most one partial 128-row
//     tile;
//   - one LDS stage is 128 bytes of K (four scale blocks): codes of the 128 A
//     rows and 256 B rows plus their 32-bit scale words, all copied straight
//     from global memory into LDS (global_load_lds, 16-byte pieces for codes,
//     4-byte pieces for scale words); three stages rotate, so the loads of
//     stage k+2 are in flight while stage k feeds the matrix cores;
//   - LDS reads are issued explicitly (ds_read_b128) one MFMA group ahead and
//     waited for with lgkmcnt just before use; one barrier per stage.
//
// Operand layout of the scaled MFMA (measured on gfx950): lane l holds row
// l % 32 (A) or column l % 32 (B) and the 16-byte K pieces [16 h, 16 h + 16)
// and [32 + 16 h, 32 + 16 h + 16) of a 64-byte K step, h = l / 32; the E8M0
// scale in byte 0 of lane l's scale operand applies to 32-block h of that row
// or column.  A lane therefore reads 16-byte chunks c0 + h and c0 + 2 + h of
// its LDS row and passes byte (2 s + h) of the row's scale word for K step s.
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

constexpr int kMxBM = 128;   // rows per tile
constexpr int kMxBN = 256;   // B rows per tile
constexpr int kMxStages = 3;

__device__ __forceinline__ void mx_barrier() { __asm__ volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ uint4 mx_ds_read16(uint32_t addr) {
    uint4 v;
    __asm__ volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr) : "memory");
    return v;
}

__device__ __forceinline__ uint32_t mx_ds_read4(uint32_t addr) {
    uint32_t v;
    __asm__ volatile("ds_read_b32 %0, %1" : "=v"(v) : "v"(addr) : "memory");
    return v;
}

template <bool SWIGLU>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_mxfp8(MxArgs p) {
    constexpr int BKB = 128;                       // K bytes per stage
    constexpr int CH = BKB / 16;                   // 16-byte chunks per LDS row
    constexpr int RPL = 64 / CH;                   // rows per wave-wide code load
    constexpr int A_LOADS = kMxBM / 4 / RPL;       // 4: each wave loads 32 A rows
    constexpr int B_LOADS = kMxBN / 4 / RPL;       // 8: each wave loads 64 B rows
    constexpr int LPS = A_LOADS + B_LOADS + 2;     // loads per wave per stage (+ two scale loads)
    constexpr int A_BYTES = kMxBM * BKB;           // 16 KiB
    constexpr int B_BYTES = kMxBN * BKB;           // 32 KiB
    constexpr int AS_OFF = A_BYTES + B_BYTES;      // scale words of the A rows
    constexpr int BS_OFF = AS_OFF + kMxBM * 4;     // scale words of the B rows
    constexpr int ST_BYTES = BS_OFF + kMxBN * 4;   // 50688
    static_assert(LPS == 14, "wait counts below");

    __shared__ __attribute__((aligned(1024))) uint8_t lds[kMxStages * ST_BYTES];
    __shared__ int32_t pre[kMaxExperts + 1];
    __shared__ int scan_tmp[kThreads / 64];

    const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wid >> 1, wn = wid & 1, half = lane >> 5;
    const int total_m = build_tile_prefix(p.offsets, p.E, kMxBM, pre, scan_tmp);
    const int cols_per_tile = SWIGLU ? kMxBN / 2 : kMxBN;
    const int n_tiles = (p.n_out + cols_per_tile - 1) / cols_per_tile;
    const int total = total_m * n_tiles;
    const int xcd = blockIdx.x % kXcds, per_xcd = gridDim.x / kXcds;
    const int lb = blockIdx.x / kXcds;
    const int t_begin = (int)((int64_t)total * xcd / kXcds), t_end = (int)((int64_t)total * (xcd + 1) / kXcds);

    const int K = p.K, KS = K / 32;  // bytes per row, scale bytes per row
    const int nk = K / BKB;
    const int lrow = lane / CH, lslot = lane % CH;

    const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void*)lds;
    // LDS rows of this lane's MFMA operands (2 x 4 accumulators of 32 x 32 per wave)
    int arow[2], brow[4];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) arow[mi] = wm * 64 + mi * 32 + (lane & 31);
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
        brow[ni] = SWIGLU ? (ni < 2 ? 0 : 128) + wn * 64 + (ni & 1) * 32 + (lane & 31)
                          : wn * 128 + ni * 32 + (lane & 31);
    // LDS byte address of fragment 0 of A and of B (stage 0), the row offsets
    // of B fragments 1..3, and the lane's chunk offsets for K step sub, half hl
    const uint32_t ra0 = lds_base + (uint32_t)arow[0] * BKB, rb0 = lds_base + A_BYTES + (uint32_t)brow[0] * BKB;
    constexpr int kBRow[4] = {0, 32, SWIGLU ? 128 : 64, SWIGLU ? 160 : 96};
    // (LDS holds chunk c of row r at position c ^ swz<1>(r): any 16
    // consecutive rows of a fragment then cover all 64 banks, so a
    // ds_read_b128 is conflict-free; fragments start at multiples of 32 rows,
    // so swz<1> of a fragment row depends only on the lane and the fragment's
    // parity par)
    uint32_t kc[2][2][2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int hl = 0; hl < 2; ++hl)
#pragma unroll
            for (int par = 0; par < 2; ++par)
                kc[sub][hl][par] = (uint32_t)(((sub * 4 + hl * 2 + half) ^ swz<1>(par * 32 + (lane & 31))) << 4);

    for (int t = t_begin + lb; t < t_end; t += per_xcd) {
        int mt, nt;
        // Tiles are ordered expert by expert, and within an expert N-tile by
        // N-tile with its M-tiles adjacent: the blocks of one XCD that run at
        // the same time then cover few experts, so each weight panel is
        // fetched from HBM once and shared in L2 by all of the expert's M-tiles.
        const int e = __builtin_amdgcn_readfirstlane(find_expert(pre, p.E, t / n_tiles));
        {
            const int m_e = pre[e + 1] - pre[e], li = t - pre[e] * n_tiles;
            nt = li / m_e;
            mt = pre[e] + li % m_e;
        }
        nt = __builtin_amdgcn_readfirstlane(nt);
        const int row_end = __builtin_amdgcn_readfirstlane(min(p.offsets[e + 1], p.rows));
        const int row0 = __builtin_amdgcn_readfirstlane(p.offsets[e] + (mt - pre[e]) * kMxBM);
        if (row0 < 0 || row0 >= row_end) continue;  // only for inconsistent offsets

        auto b_row_of = [&](int r) __attribute__((always_inline)) {
            if (SWIGLU) {
                const int f = min(nt * 128 + (r & 127), p.n_out - 1);
                return r < 128 ? f : p.n_out + f;
            }
            return min(nt * kMxBN + r, p.n_out - 1);
        };
        // per-lane global byte offsets of the code loads (K offset 0); the
        // 16-byte chunk a lane fetches is permuted so that LDS holds chunk
        // c of row r at position c ^ swz<1>(r) (conflict-free fragment reads)
        uint32_t aoff[A_LOADS], boff[B_LOADS];
#pragma unroll
        for (int i = 0; i < A_LOADS; ++i) {
            const int r = wid * 32 + i * RPL + lrow;
            aoff[i] = (uint32_t)((size_t)(min(row0 + r, row_end - 1) - row0) * K + ((lslot ^ swz<1>(r)) * 16));
        }
#pragma unroll
        for (int i = 0; i < B_LOADS; ++i) {
            const int r = wid * 64 + i * RPL + lrow;
            boff[i] = (uint32_t)((size_t)b_row_of(r) * K + ((lslot ^ swz<1>(r)) * 16));
        }
        const uint8_t* acodes = p.A + (size_t)row0 * K;  // A offsets are tile-relative
        const uint8_t* bcodes = p.B + (size_t)e * p.b_rows * K;
        // scale words: A rows wid*32 + lane (lanes 0..31), B rows wid*64 + lane,
        // as uniform bases plus 32-bit lane offsets
        const uint8_t* asbase = p.As + (size_t)row0 * KS;
        const uint8_t* bsbase = p.Bs + (size_t)e * p.b_rows * KS;
        const uint32_t asoff = (uint32_t)((min(row0 + wid * 32 + (lane & 31), row_end - 1) - row0) * KS);
        const uint32_t bsoff = (uint32_t)(b_row_of(wid * 64 + lane) * KS);

        f32x16 acc[2][4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

        // Loads of stage kt into stage buffer slot % 3 (dma_lds16 / dma_lds4:
        // uniform M0 and base, 32-bit lane offsets): the codes of this wave's
        // 32 A rows (4 loads) and 64 B rows (8 loads), and the 32-bit scale
        // words of those rows (one load each).  MX_LD(slot, kt, j) is load j
        // of 14; slot = kt except past the end of K, where the last stage is
        // loaded again into the free buffer.
#define MX_LD(slot, kt, j)                                                                               \
    {                                                                                                    \
        const uint32_t st_ = lds_base + (uint32_t)((slot) % kMxStages) * ST_BYTES;                       \
        if ((j) < A_LOADS)                                                                               \
            dma_lds16(__builtin_amdgcn_readfirstlane(st_ + (wid * 32 + (j) * RPL) * BKB), aoff[(j) % A_LOADS], \
                      acodes + (size_t)(kt) * BKB);                                                      \
        else if ((j) < A_LOADS + B_LOADS)                                                                \
            dma_lds16(__builtin_amdgcn_readfirstlane(st_ + A_BYTES + (wid * 64 + ((j) - A_LOADS) * RPL) * BKB), \
                      boff[((j) - A_LOADS) % B_LOADS], bcodes + (size_t)(kt) * BKB);                      \
        else if ((j) == A_LOADS + B_LOADS) {                                                             \
            if (lane < 32)                                                                               \
                dma_lds4(__builtin_amdgcn_readfirstlane(st_ + AS_OFF + wid * 32 * 4), asoff, asbase + (size_t)(kt) * 4); \
        } else                                                                                           \
            dma_lds4(__builtin_amdgcn_readfirstlane(st_ + BS_OFF + wid * 64 * 4), bsoff, bsbase + (size_t)(kt) * 4); \
    }
#define MX_ISSUE(kt)                                                                                     \
    _Pragma("unroll") for (int j_ = 0; j_ < LPS; ++j_) MX_LD(kt, kt, j_)
        // Fragment reads of K step `sub` (64 bytes) of the stage at byte offset
        // so_: A fragment mi / B fragment ni from 16-byte chunks 4 sub + h and
        // 4 sub + 2 + h of the lane's row (h = lane / 32), stored at chunk
        // position c ^ swz<1>(row) (kc, by the fragment's parity).
#define MX_RD_A(FA, so_, sub, mi)                                                                        \
    {                                                                                                    \
        const uint4 lo_ = mx_ds_read16(ra0 + (so_) + kc[sub][0][(mi) & 1] + (mi) * 32 * BKB);                      \
        const uint4 hi_ = mx_ds_read16(ra0 + (so_) + kc[sub][1][(mi) & 1] + (mi) * 32 * BKB);                      \
        FA[mi] = i32x8{(int)lo_.x, (int)lo_.y, (int)lo_.z, (int)lo_.w, (int)hi_.x, (int)hi_.y, (int)hi_.z, (int)hi_.w}; \
    }
#define MX_RD_B(FB, so_, sub, ni)                                                                        \
    {                                                                                                    \
        const uint4 lo_ = mx_ds_read16(rb0 + (so_) + kc[sub][0][(ni) & 1] + kBRow[ni] * BKB);                      \
        const uint4 hi_ = mx_ds_read16(rb0 + (so_) + kc[sub][1][(ni) & 1] + kBRow[ni] * BKB);                      \
        FB[ni] = i32x8{(int)lo_.x, (int)lo_.y, (int)lo_.z, (int)lo_.w, (int)hi_.x, (int)hi_.y, (int)hi_.z, (int)hi_.w}; \
    }
        // the 32-bit scale words (one byte per 32 K values of the stage) of the lane's rows
#define MX_RD_S(SA, SB, so_)                                                                             \
    {                                                                                                    \
        _Pragma("unroll") for (int mi = 0; mi < 2; ++mi) SA[mi] = mx_ds_read4(lds_base + (so_) + AS_OFF + arow[mi] * 4); \
        _Pragma("unroll") for (int ni = 0; ni < 4; ++ni) SB[ni] = mx_ds_read4(lds_base + (so_) + BS_OFF + brow[ni] * 4); \
    }
#define MX_WAIT(FA, FB)                                                                                  \
    __asm__ volatile("s_waitcnt lgkmcnt(0)"                                                              \
                     : "+v"(FA[0]), "+v"(FA[1]), "+v"(FB[0]), "+v"(FB[1]), "+v"(FB[2]), "+v"(FB[3])::"memory")
#define MX_WAIT_S(SA, SB)                                                                                \
    __asm__ volatile("s_waitcnt lgkmcnt(0)"                                                              \
                     : "+v"(SA[0]), "+v"(SA[1]), "+v"(SB[0]), "+v"(SB[1]), "+v"(SB[2]), "+v"(SB[3])::"memory")
        // One MFMA of K step SUB: the scale words were shifted right by 8 h, so
        // the byte of 32-block 2 SUB + h is byte 2 SUB for every lane (opsel).
#define MX_MFMA(FA, FB, SA, SB, SUB, mi, ni)                                                             \
    acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(FA[mi], FB[ni], acc[mi][ni], 0, 0, 2 * (SUB), \
                                                                  (int)SA[mi], 2 * (SUB), (int)SB[ni])
#define MX_SB __builtin_amdgcn_sched_barrier(0)
#define MX_STEP(PRE, MF, RD)                                                                             \
    PRE;                                                                                                 \
    MF;                                                                                                  \
    RD;                                                                                                  \
    MX_SB;

        const int KT_ = nk;  // stages
        // prologue: stages 0 and 1 in flight, stage 0 landed everywhere
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");  // previous tile's stores retired
        MX_SB;
        MX_ISSUE(0);
        _Pragma("unroll") for (int j_ = 0; j_ < LPS; ++j_) MX_LD(1, min(1, KT_ - 1), j_)
        __asm__ volatile("s_waitcnt vmcnt(14)\n\ts_barrier" ::: "memory");
        MX_SB;
        i32x8 f0a[2], f0b[4], f1a[2], f1b[4];
        uint32_t s0a[2], s0b[4], s1a[2], s1b[4];
        MX_RD_A(f0a, 0u, 0, 0) MX_RD_A(f0a, 0u, 0, 1)
        MX_RD_B(f0b, 0u, 0, 0) MX_RD_B(f0b, 0u, 0, 1) MX_RD_B(f0b, 0u, 0, 2) MX_RD_B(f0b, 0u, 0, 3)
        MX_RD_S(s1a, s1b, 0u)
        for (int kt = 0; kt < KT_; ++kt) {
            const uint32_t so = (uint32_t)(kt % kMxStages) * ST_BYTES;
            const uint32_t sn = (uint32_t)((kt + 1) % kMxStages) * ST_BYTES;
            const int kl = min(kt + 2, KT_ - 1);  // loads of stage kt+2 (past the end: the last stage again)
            MX_SB;
            // this stage's scale words, shifted so byte 2 s holds 32-block 2 s + h
            MX_WAIT_S(s1a, s1b);
#pragma unroll
            for (int i = 0; i < 2; ++i) s0a[i] = s1a[i] >> (8 * half);
#pragma unroll
            for (int i = 0; i < 4; ++i) s0b[i] = s1b[i] >> (8 * half);
            MX_WAIT(f0a, f0b);
            MX_SB;
            // K step 0: 8 MFMAs; the fragments of step 1 and loads 0..6 of stage kt+2 ride along
            MX_STEP(MX_LD(kt + 2, kl, 0), MX_MFMA(f0a, f0b, s0a, s0b, 0, 0, 0), MX_RD_A(f1a, so, 1, 0))
            MX_STEP(MX_LD(kt + 2, kl, 1), MX_MFMA(f0a, f0b, s0a, s0b, 0, 0, 1), MX_RD_A(f1a, so, 1, 1))
            MX_STEP(MX_LD(kt + 2, kl, 2), MX_MFMA(f0a, f0b, s0a, s0b, 0, 0, 2), MX_RD_B(f1b, so, 1, 0))
            MX_STEP(MX_LD(kt + 2, kl, 3), MX_MFMA(f0a, f0b, s0a, s0b, 0, 0, 3), MX_RD_B(f1b, so, 1, 1))
            MX_STEP(MX_LD(kt + 2, kl, 4), MX_MFMA(f0a, f0b, s0a, s0b, 0, 1, 0), MX_RD_B(f1b, so, 1, 2))
            MX_STEP(MX_LD(kt + 2, kl, 5), MX_MFMA(f0a, f0b, s0a, s0b, 0, 1, 1), MX_RD_B(f1b, so, 1, 3))
            MX_STEP(MX_LD(kt + 2, kl, 6), MX_MFMA(f0a, f0b, s0a, s0b, 0, 1, 2), (void)0)
            MX_STEP((void)0, MX_MFMA(f0a, f0b, s0a, s0b, 0, 1, 3), (void)0)
            MX_WAIT(f1a, f1b);  // this wave has read all of stage kt
            // stage kt+1 landed (only the 7 loads of stage kt+2 just issued may
            // be in flight); past the barrier the same holds for every wave and
            // the buffer of stage kt is free
            __asm__ volatile("s_waitcnt vmcnt(7)\n\ts_barrier" ::: "memory");
            MX_SB;
            // K step 1: 8 MFMAs; step 0 and the scale words of stage kt+1 and
            // loads 7..13 of stage kt+2 ride along
            MX_STEP(MX_LD(kt + 2, kl, 7), MX_MFMA(f1a, f1b, s0a, s0b, 1, 0, 0), MX_RD_A(f0a, sn, 0, 0))
            MX_STEP(MX_LD(kt + 2, kl, 8), MX_MFMA(f1a, f1b, s0a, s0b, 1, 0, 1), MX_RD_A(f0a, sn, 0, 1))
            MX_STEP(MX_LD(kt + 2, kl, 9), MX_MFMA(f1a, f1b, s0a, s0b, 1, 0, 2), MX_RD_B(f0b, sn, 0, 0))
            MX_STEP(MX_LD(kt + 2, kl, 10), MX_MFMA(f1a, f1b, s0a, s0b, 1, 0, 3), MX_RD_B(f0b, sn, 0, 1))
            MX_STEP(MX_LD(kt + 2, kl, 11), MX_MFMA(f1a, f1b, s0a, s0b, 1, 1, 0), MX_RD_B(f0b, sn, 0, 2))
            MX_STEP(MX_LD(kt + 2, kl, 12), MX_MFMA(f1a, f1b, s0a, s0b, 1, 1, 1), MX_RD_B(f0b, sn, 0, 3))
            MX_STEP(MX_LD(kt + 2, kl, 13), MX_MFMA(f1a, f1b, s0a, s0b, 1, 1, 2), MX_RD_S(s1a, s1b, sn))
            MX_STEP((void)0, MX_MFMA(f1a, f1b, s0a, s0b, 1, 1, 3), (void)0)
            // wait for the next stage's step-0 fragments and scale words here
            // (they had the last MFMAs to land), so no LDS read is in flight
            // when the loop ends
            MX_WAIT(f0a, f0b);
            MX_WAIT_S(s1a, s1b);
        }
        MX_SB;
        // every wave passed the last barrier after reading its last stage, and
        // its last loads (repeats of the last stage) went to the free buffer
        __asm__ volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");  // LDS free for the epilogue
#undef MX_LD
#undef MX_ISSUE
#undef MX_RD_A
#undef MX_RD_B
#undef MX_RD_S
#undef MX_WAIT
#undef MX_WAIT_S
#undef MX_MFMA
#undef MX_SB
#undef MX_STEP
        // every wave passed the last barrier after reading its last stage: LDS is free

        // epilogue through LDS: lane -> row rr, columns cc .. cc+15 of a 32x32 tile
        float* wb = (float*)lds + wid * 2 * (32 * 33 + 32);
        float* wb2 = wb + 32 * 33 + 32;
        const int rr = lane >> 1, cc = (lane & 1) * 16;
        if (SWIGLU) {
#define GM_EPI_SW(MI, NI)                                                                                \
    {                                                                                                    \
        GE_STAGE_TILE(wb, acc[MI][NI])                                                                   \
        GE_STAGE_TILE(wb2, acc[MI][(NI) + 2])                                                            \
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
        const int r = row0 + wm * 64 + (MI) * 32 + rr;                                                   \
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
                    gs[j] = GE_PACK8(gv, 8 * j);                                                         \
                    us[j] = GE_PACK8(uv, 8 * j);                                                         \
                }                                                                                        \
            }                                                                                            \
        }                                                                                                \
    }
            GM_EPI_SW(0, 0) GM_EPI_SW(0, 1) GM_EPI_SW(1, 0) GM_EPI_SW(1, 1)
#undef GM_EPI_SW
        } else {
#define GM_EPI_DN(MI, NI)                                                                                \
    {                                                                                                    \
        GE_STAGE_TILE(wb, acc[MI][NI])                                                                   \
        __builtin_amdgcn_s_waitcnt(0xC07F);                                                              \
        float v[16];                                                                                     \
        _Pragma("unroll") for (int j = 0; j < 16; ++j) v[j] = wb[rr * 33 + cc + j];                      \
        __builtin_amdgcn_s_waitcnt(0xC07F);                                                              \
        const int r = row0 + wm * 64 + (MI) * 32 + rr;                                                   \
        const int n = nt * kMxBN + wn * 128 + (NI) * 32 + cc;                                            \
        if (r < row_end && n < p.n_out) {                                                                \
            uint4* dst = (uint4*)(p.Cb + (size_t)r * p.n_out + n);                                       \
            _Pragma("unroll") for (int j = 0; j < 2; ++j) dst[j] = GE_PACK8(v, 8 * j);                  \
        }                                                                                                \
    }
            GM_EPI_DN(0, 0) GM_EPI_DN(0, 1) GM_EPI_DN(0, 2) GM_EPI_DN(0, 3)
            GM_EPI_DN(1, 0) GM_EPI_DN(1, 1) GM_EPI_DN(1, 2) GM_EPI_DN(1, 3)
#undef GM_EPI_DN
        }
        __syncthreads();  // LDS reused by the next tile's loads
    }
}

}  // namespace gemm
}  // namespace moe
