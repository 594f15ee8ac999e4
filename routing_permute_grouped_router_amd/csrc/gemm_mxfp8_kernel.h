// Grouped MXFP8 and MXFP4 GEMMs on CDNA4 scaled matrix cores
// (v_mfma_scale_f32_32x32x64_f8f6f4; E4M3 or E2M1 operands, E8M0 scales per 32).
//
// Same computation and device-side group handling as the bf16 kernel
// (gemm_bf16_kernel.h), on the MXFP8 block-scaled format of the cudnn-frontend
// page "Add MoE + expert-parallel Python API surface, PyTorch reference, and
// tests" (BlockScaledTensor, block 32) with OCP E4M3 elements.
//
// Operand layout of the scaled MFMA (measured on gfx950): lane l holds row
// l % 32 (A) or column l % 32 (B) and the 16-byte K pieces [16 h, 16 h + 16)
// and [32 + 16 h, 32 + 16 h + 16) of a 64-byte K step, h = l / 32; the E8M0
// scale in byte 0 of lane l's scale operand applies to 32-block h of that row
// or column.  A lane therefore reads 16-byte chunks 4 s + h and 4 s + 2 + h of
// its LDS row and passes byte (2 s + h) of the row's scale word for K step s.
//
// MXFP4 (F4): the same instruction with E2M1 operands reads 4 registers per
// lane, all 32 values of one scale block: lane l holds row (column) l % 32
// and 32-block h = l / 32 of a 64-value K step, and its scale operand gives
// that block's scale (measured on gfx950).  A 16-byte chunk of a packed row
// is exactly one block, so the chunks 4 s + h and 4 s + 2 + h that the E4M3
// form reads as one 64-byte K step are two E2M1 K steps here: one MFMA on
// the low four registers (block 4 s + h, scale byte 0 after the shift) and
// one on the high four (block 4 s + 2 + h, scale byte 2).  A 128-byte stage
// holds 256 values (8 blocks, two scale words per row), so every LDS read
// feeds twice the MFMA work of the E4M3 form.
#pragma once

#include "gemm_bf16_kernel.h"
#include "mxfp8.h"

namespace moe {
namespace gemm {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// The scaled MFMA with 4-register (E2M1) operands: the LLVM intrinsic's
// 128-bit overload, which the clang builtin (8-register operands only) does
// not expose.  cbsz / blgp 4 select E2M1 for A / B; opsel picks the scale byte.
__device__ f32x16 mfma_scale_e2m1(i32x4 a, i32x4 b, f32x16 c, int cbsz, int blgp, int opsel_a, int scale_a,
                                  int opsel_b, int scale_b)
    __asm("llvm.amdgcn.mfma.scale.f32.32x32x64.f8f6f4.v4i32.v4i32");

struct MxArgs {
    const uint8_t* A;        // [rows][K] E4M3 codes (MXFP4: [rows][K/2], two E2M1 per byte)
    const uint8_t* As;       // [rows][K/32] E8M0 scales
    const uint8_t* B;        // [E][b_rows][K]
    const uint8_t* Bs;       // [E][b_rows][K/32]
    const int32_t* offsets;  // [E+1]
    int E, K, rows, n_out, b_rows;  // K: elements
    uint8_t* C;              // SwiGLU: h codes [rows][n_out] (MXFP4: [rows][n_out/2])
    uint8_t* Cs;             // SwiGLU: h scales [rows][n_out/32]
    uint16_t* Cb;            // down: Yp bf16 [rows][n_out]
    uint16_t* stash;         // SwiGLU, optional: bf16 g | u [rows][2 n_out]
    int* sched;              // 8 work-queue counters, zero at launch
    // gather (SwiGLU only; src_map null otherwise): A / As are x codes / scales
    // [T, K], row r of the grouped operand is x[src_map[r] / gk]; the first
    // counts[e] rows of expert e are routed, the rest are padding rows, whose h
    // is stored as zeros (codes 0, scale code 0, as for zero rows of Xp)
    const int32_t* src_map;
    const int32_t* counts;
    int gk;
    // optional per-row routing weights (the epilogue placements of the
    // weight): output row r is scaled by row_w[r] before it is stored (h
    // before its quantisation); 256 rows past `rows` are readable
    const float* row_w;
    // SwiGLU clamp limit (the clamped variant only): g <- min(g, lim),
    // u <- clamp(u, -lim, lim) before the activation; +inf when off
    float lim;
};

// ---------------------------------------------------------------------------
// 256 x 256 tiles.  Each wavefront owns a 128 x 128 sub-tile (4 x 4 scaled
// MFMAs), so every operand fragment read from LDS feeds two MFMAs (a 64 x 128
// wavefront tile feeds 1.33 and needs ~100 bytes of fragment reads per MFMA
// cycle and CU, near what LDS serves; here 64).
// Two stages of 128 K-bytes of E4M3 codes rotate through LDS; a stage is two
// K steps of 16 MFMAs each (2048 cycles, as long as a stage of the bf16
// kernel).  Two barriers per stage.  The first, after the first K step, only
// needs every wavefront to have read all of stage kt: its buffer is free, and
// the 16 code loads of stage kt+2 go into it under the 16 MFMAs of the second
// K step, four of B first.  The second, after those four, needs stage kt+1 to
// have landed (vmcnt(4): only those four loads are younger, and vector memory
// operations complete in issue order); the fragments of stage kt+1's first K
// step and its scale words are read after it.  Waiting for stage kt+1 there
// rather than at the first barrier gives its last loads four more MFMAs (256
// cycles) to land.  Scale words (one 32-bit word of four E8M0 bytes per
// row and stage) sit in two slots of their own: with K a multiple of 512, a
// 16-byte load per row brings the words of four stages (a row's scales are
// 224 bytes apart at K = 7168, so each 4-byte load touched its own cache
// line: as many L2 requests as all the code loads); else one word per stage.  Scheduling as in the bf16 kernel: per-XCD work queues
// with stealing, the next unit's first stage and a half issued before the
// epilogue (no K split: its partial sums would need the requantising
// epilogue in a second kernel).
//
// Epilogues.  Down GEMM: bf16 straight from the accumulators with the
// column order of the B rows chosen so that each lane stores 8-byte words of
// four adjacent columns (out_col).  SwiGLU GEMM: h = silu(g) u is formed in
// registers and each 32 x 32 h tile goes through a wavefront-private LDS tile
// so that each lane finishes 16 consecutive columns of one row: the two
// lanes of a 32-block exchange their partial maxima, quantise to E4M3
// (OCP rule) and store 16 bytes of codes plus the scale byte.  The LDS tile
// of wavefront w is the part of stage buffer 1 that only w's own loads write
// (its 64 B-code rows): the next unit's B half of that buffer is issued only
// after the epilogue, once w's reads of the tile are done.

// A copy of a wavefront-uniform value that the compiler cannot see through,
// so that a compare on it is made where it is used (a scalar compare and
// branch) rather than hoisted out of the loop as a lane mask.
__device__ __forceinline__ int opaque_s(int v) {
    __asm__ volatile("" : "+s"(v));
    return v;
}

// One operand fragment of a 64-byte K step: two 16-byte chunks (lo, hi).
template <int OFF>
__device__ __forceinline__ i32x8 mx_frag(uint32_t lo, uint32_t hi) {
    uint4 a, b;
    __asm__ volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(a) : "v"(lo), "i"(OFF) : "memory");
    __asm__ volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(b) : "v"(hi), "i"(OFF) : "memory");
    return i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}
template <int OFF>
__device__ __forceinline__ uint32_t mx_word(uint32_t addr) {
    uint32_t v;
    __asm__ volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF) : "memory");
    return v;
}
template <int OFF>
__device__ __forceinline__ uint2 mx_word2(uint32_t addr) {
    uint2 v;
    __asm__ volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF) : "memory");
    return v;
}

// EP, epilogue variant bits (built separately, so the plain kernel carries
// none of it): 1 = the outputs are scaled by p.row_w, 2 = the SwiGLU inputs
// are clamped to p.lim.  F4: E2M1 operands (and h) instead of E4M3.
template <bool SWIGLU, int G, int EP, bool F4>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_mxfp8(MxArgs p) {
    constexpr int BKB = 128;                 // K bytes per stage: 128 E4M3 values (4 blocks) or 256 E2M1 (8)
    constexpr int CH = BKB / 16;             // 16-byte chunks per LDS row
    constexpr int RPL = 64 / CH;             // rows per wave-wide code load
    constexpr int LOADS = 64 / RPL;          // code loads per wave per operand per stage
    constexpr int OPB = kTile * BKB;         // codes of one operand in one stage (32 KiB)
    constexpr uint32_t STB = 2 * OPB;        // one stage: A codes | B codes
    // Scale words: G stages per load (16 bytes per row, one cache line per row
    // every G stages instead of every stage: G = 4 for E4M3, whose stage has
    // one word per row, and G = 2 for E2M1, two words; G = 1: one 4-byte
    // E4M3 word per stage), in two slots of [A rows | B rows] x SWB G bytes
    // after the two stages; stage kt's words of row r are at slot (kt / G) % 2,
    // byte SWB (kt % G) of the row's entry.
    constexpr int SWB = F4 ? 8 : 4;  // scale bytes per row and stage
    static_assert(F4 ? G == 2 : (G == 1 || G == 4), "scale group");
    constexpr int SW_ROW = SWB * G, SC_OP = kTile * SW_ROW, SC_SLOT = 2 * SC_OP;
    constexpr uint32_t SC_BASE = 2 * STB;
    // byte offsets of B fragments 1..3 from fragment 0 (SwiGLU: fragments 2, 3
    // are the up rows of fragments 0, 1)
    constexpr int B1 = 32 * BKB, B2 = (SWIGLU ? 128 : 64) * BKB, B3 = (SWIGLU ? 160 : 96) * BKB;
    constexpr int W1 = 32 * SW_ROW, W2 = (SWIGLU ? 128 : 64) * SW_ROW, W3 = (SWIGLU ? 160 : 96) * SW_ROW;

    __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * STB + 2 * SC_SLOT];
    __shared__ int32_t pre[kMaxExperts + 1];
    __shared__ int32_t offs[kMaxExperts + 1];
    __shared__ int scan_tmp[kThreads / 64];
    __shared__ Queue queues[kXcds];
    __shared__ int s_unit;

    const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wid >> 1, wn = wid & 1, half = lane >> 5;
    for (int e = tid; e <= p.E; e += kThreads) offs[e] = p.offsets[e];
    const int total_m = build_tile_prefix(p.offsets, p.E, kTile, pre, scan_tmp);  // ends with a barrier
    const int cols_per_tile = SWIGLU ? kTile / 2 : kTile;
    const int n_tiles = (p.n_out + cols_per_tile - 1) / cols_per_tile;
    const int total = total_m * n_tiles;
    const int K = p.K, KS = K / 32, KB = F4 ? K / 2 : K, nk = KB / BKB;  // KB: bytes per row
    const int xcd = blockIdx.x % kXcds, nb = gridDim.x / kXcds;
    if (tid < kXcds) queues[tid] = xcd_queue(total, tid, nb, 0);  // whole tiles only
    uint32_t dry = 0;
    auto ticket = [&]() -> int { return (dry >> xcd & 1) ? -1 : atomicAdd(p.sched + xcd, 1); };
    auto take = [&](int r) -> int {
        if (!(dry >> xcd & 1)) {
            if (r >= 0 && r < queues[xcd].units) return (xcd << 20) | r;
            dry |= 1u << xcd;
        }
        for (int d = 1; d < kXcds; ++d) {
            const int x = (xcd + d) % kXcds;
            if (dry >> x & 1) continue;
            const int u = atomicAdd(p.sched + x, 1);
            if (u < queues[x].units) return (x << 20) | u;
            dry |= 1u << x;
        }
        return -1;
    };
    __syncthreads();
    int tick = -1;
    if (tid == 0) {
        s_unit = take(ticket());
        tick = ticket();
    }
    __syncthreads();
    int unit = s_unit;

    const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void*)&lds[0];
    // LDS rows this wave's loads fill: wid * 64 .. +63 of each operand
    const uint32_t lds_wave = __builtin_amdgcn_readfirstlane(lds_base + (uint32_t)(wid * 64 * BKB));
    const uint32_t lds_wsc = __builtin_amdgcn_readfirstlane(lds_base + SC_BASE + (uint32_t)(wid * 64 * SW_ROW));
    const int bfr = SWIGLU ? wn * 64 : wn * 128;  // first B row of this wave's fragments
    // the wavefront's A fragment mi is tile rows 32 (2 mi + wm) .. + 31
    const uint32_t a_rd = lds_base + (uint32_t)((wm * 32 + (lane & 31)) * BKB);
    const uint32_t b_rd = lds_base + (uint32_t)(OPB + (bfr + (lane & 31)) * BKB);
    const uint32_t as_rd = lds_base + SC_BASE + (uint32_t)((wm * 32 + (lane & 31)) * SW_ROW);
    const uint32_t bs_rd = lds_base + SC_BASE + (uint32_t)(SC_OP + (bfr + (lane & 31)) * SW_ROW);
    // chunk offsets [K step][lo, hi][fragment parity]: lane l reads 16-byte
    // chunks 4 s + h and 4 s + 2 + h (h = l / 32) of row l % 32 of a
    // fragment, stored at position c ^ swz<1>(row)
    uint32_t kc[2][2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int hl = 0; hl < 2; ++hl)
#pragma unroll
            for (int par = 0; par < 2; ++par)
                kc[s][hl][par] = (uint32_t)(((4 * s + 2 * hl + half) ^ swz<1>(par * 32 + (lane & 31))) << 4);
    // the same for the A fragments, all of whose rows have parity wm
    uint32_t kca[2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int hl = 0; hl < 2; ++hl)
            kca[s][hl] = (uint32_t)(((4 * s + 2 * hl + half) ^ swz<1>(wm * 32 + (lane & 31))) << 4);

    int kb = 0, ke = 0, row0 = 0, row_end = 0, a_end = 0, nt = 0;
    // this wavefront's A fragments with rows of the group (nv, 0..4), and its
    // A code loads per stage that fill rows of the tile's fragments with rows
    // (na, 0..LOADS)
    int nv = 4, na = LOADS;
    bool valid = false;
    uint32_t aoff[LOADS], boff[LOADS], asoff = 0, bsoff = 0;
    const uint8_t* acodes = p.A;
    const uint8_t* bcodes = p.B;
    const uint8_t* ascale = p.As;
    const uint8_t* bscale = p.Bs;
#define MX_LOAD_A(kt, stage, i)                                                                          \
    dma_lds16(lds_wave + (uint32_t)(stage) * STB + (i) * RPL * BKB, aoff[i], acodes + (size_t)(kt) * BKB)
// an in-loop A load, skipped when it fills only rows of fragments without rows
#define MX_LOAD_A_IF(kt, stage, i)                                                                       \
    if ((i) < opaque_s(na)) MX_LOAD_A(kt, stage, i)
#define MX_LOAD_B(kt, stage, i)                                                                          \
    dma_lds16(lds_wave + (uint32_t)(stage) * STB + OPB + (i) * RPL * BKB, boff[i], bcodes + (size_t)(kt) * BKB)
// scale words of load group grp (G stages) into slot `slot`
#define MX_LOAD_SC(OP, SOFF, SBASE, grp, slot)                                                           \
    {                                                                                                    \
        if constexpr (G * SWB == 16)                                                                     \
            dma_lds16(lds_wsc + (uint32_t)(slot) * SC_SLOT + (OP) * SC_OP, SOFF, SBASE + (size_t)(grp) * 16); \
        else                                                                                             \
            dma_lds4(lds_wsc + (uint32_t)(slot) * SC_SLOT + (OP) * SC_OP, SOFF, SBASE + (size_t)(grp) * 4); \
    }
#define MX_LOAD_AS(grp, slot) MX_LOAD_SC(0, asoff, ascale, grp, slot)
#define MX_LOAD_BS(grp, slot) MX_LOAD_SC(1, bsoff, bscale, grp, slot)
// LDS byte offset of stage kt's scale words within the scale slots
#define MX_SC_OFF(kt) ((uint32_t)(((kt) / G) & 1) * SC_SLOT + (uint32_t)((kt) % G) * SWB)
#define MX_SB __builtin_amdgcn_sched_barrier(0)
// fragment reads of K step S of the stage at byte offset SO
#define MX_RD_A(F, SO, S, mi)                                                                            \
    F[mi] = mx_frag<(mi) * 64 * BKB>(a_rd + (SO) + kca[S][0], a_rd + (SO) + kca[S][1])
#define MX_RD_B(G, SO, S, ni)                                                                            \
    G[ni] = mx_frag<(ni) == 0 ? 0 : (ni) == 1 ? B1 : (ni) == 2 ? B2 : B3>(b_rd + (SO) + kc[S][0][(ni) & 1], \
                                                                          b_rd + (SO) + kc[S][1][(ni) & 1])
// the scale words of a stage (SO = MX_SC_OFF of the stage): A rows of
// fragments 0..3, then B; E2M1: the two words of fragment row i in sw2[i]
#define MX_RD_S(SW, SO)                                                                                  \
    {                                                                                                    \
        if constexpr (F4) {                                                                              \
            sw2[0] = mx_word2<0>(as_rd + (SO));                                                          \
            sw2[1] = mx_word2<64 * SW_ROW>(as_rd + (SO));                                                \
            sw2[2] = mx_word2<128 * SW_ROW>(as_rd + (SO));                                               \
            sw2[3] = mx_word2<192 * SW_ROW>(as_rd + (SO));                                               \
            sw2[4] = mx_word2<0>(bs_rd + (SO));                                                          \
            sw2[5] = mx_word2<W1>(bs_rd + (SO));                                                         \
            sw2[6] = mx_word2<W2>(bs_rd + (SO));                                                         \
            sw2[7] = mx_word2<W3>(bs_rd + (SO));                                                         \
        } else {                                                                                         \
            SW[0] = mx_word<0>(as_rd + (SO));                                                            \
            SW[1] = mx_word<64 * SW_ROW>(as_rd + (SO));                                                  \
            SW[2] = mx_word<128 * SW_ROW>(as_rd + (SO));                                                 \
            SW[3] = mx_word<192 * SW_ROW>(as_rd + (SO));                                                 \
            SW[4] = mx_word<0>(bs_rd + (SO));                                                            \
            SW[5] = mx_word<W1>(bs_rd + (SO));                                                           \
            SW[6] = mx_word<W2>(bs_rd + (SO));                                                           \
            SW[7] = mx_word<W3>(bs_rd + (SO));                                                           \
        }                                                                                                \
    }

#define MX_WAIT_F(F, G)                                                                                  \
    __asm__ volatile("s_waitcnt lgkmcnt(0)"                                                              \
                     : "+v"(F[0]), "+v"(F[1]), "+v"(F[2]), "+v"(F[3]), "+v"(G[0]), "+v"(G[1]), "+v"(G[2]), \
                       "+v"(G[3])::"memory")
#define MX_WAIT_W(SW)                                                                                    \
    {                                                                                                    \
        if constexpr (F4)                                                                                \
            __asm__ volatile("s_waitcnt lgkmcnt(0)"                                                      \
                             : "+v"(sw2[0]), "+v"(sw2[1]), "+v"(sw2[2]), "+v"(sw2[3]), "+v"(sw2[4]),    \
                               "+v"(sw2[5]), "+v"(sw2[6]), "+v"(sw2[7])::"memory");                      \
        else                                                                                             \
            __asm__ volatile("s_waitcnt lgkmcnt(0)"                                                      \
                             : "+v"(SW[0]), "+v"(SW[1]), "+v"(SW[2]), "+v"(SW[3]), "+v"(SW[4]), "+v"(SW[5]), \
                               "+v"(SW[6]), "+v"(SW[7])::"memory");                                      \
    }
// One MFMA of K step S: the scale words were shifted right by 8 h (h = lane
// / 32), so byte 2 S holds the scale of 32-block 2 S + h for every lane.
// E2M1: two MFMAs on the fragments' low and high four registers (blocks
// 4 S + h and 4 S + 2 + h: bytes 0 and 2 of the stage's word S).
#define MX_MFMA(F, G, SS, S, mi, ni)                                                                     \
    if ((mi) >= opaque_s(nv)) {                                                                          \
    } else if constexpr (F4) {                                                                           \
        acc[mi][ni] = mfma_scale_e2m1(__builtin_shufflevector(F[mi], F[mi], 0, 1, 2, 3),                 \
                                      __builtin_shufflevector(G[ni], G[ni], 0, 1, 2, 3), acc[mi][ni], 4, 4, 0, \
                                      (int)SS[2 * (mi) + (S)], 0, (int)SS[2 * (4 + (ni)) + (S)]);        \
        acc[mi][ni] = mfma_scale_e2m1(__builtin_shufflevector(F[mi], F[mi], 4, 5, 6, 7),                 \
                                      __builtin_shufflevector(G[ni], G[ni], 4, 5, 6, 7), acc[mi][ni], 4, 4, 2, \
                                      (int)SS[2 * (mi) + (S)], 2, (int)SS[2 * (4 + (ni)) + (S)]);        \
    } else {                                                                                             \
        acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F[mi], G[ni], acc[mi][ni], 0, 0, 2 * (S), \
                                                                      (int)SS[mi], 2 * (S), (int)SS[4 + (ni)]); \
    }
#define MX_STEP(F, G, SS, S, mi, ni, PRE, RD)                                                            \
    PRE;                                                                                                 \
    MX_MFMA(F, G, SS, S, mi, ni);                                                                        \
    RD;                                                                                                  \
    MX_SB;

    // Decode unit u, compute its tile's addressing and issue the loads of its
    // first stage and the A half of its second (stage buffers 0 and 1).
    auto setup = [&](int u) __attribute__((always_inline)) {
        u = __builtin_amdgcn_readfirstlane(u);
        if (u < 0) {  // no unit (every queue used up): nothing to decode or load
            valid = false;
            kb = ke = 0;
            return;
        }
        const int ux = __builtin_amdgcn_readfirstlane(u >> 20), uu = __builtin_amdgcn_readfirstlane(u & 0xFFFFF);
        const int t = __builtin_amdgcn_readfirstlane(queues[ux].tb + uu);
        kb = 0;
        ke = nk;
        int mt, ntt, ee;
        tile_of(t, pre, p.E, total_m, n_tiles, 0, &ee, &mt, &ntt);
        nt = __builtin_amdgcn_readfirstlane(ntt);
        mt = __builtin_amdgcn_readfirstlane(mt);
        const int e = __builtin_amdgcn_readfirstlane(ee);
        row_end = __builtin_amdgcn_readfirstlane(min(offs[e + 1], p.rows));
        row0 = __builtin_amdgcn_readfirstlane(offs[e] + (mt - pre[e]) * kTile);
        valid = row0 >= 0 && row0 < row_end;  // false only for inconsistent offsets
        if (!valid) {
            kb = ke = 0;
            return;
        }
        // rows with an A row of their own: all, or (gather) the routed rows
        a_end = p.src_map ? __builtin_amdgcn_readfirstlane(min(offs[e] + p.counts[e], row_end)) : row_end;
        {
            const int nfrag = (min(row_end - row0, kTile) + 31) >> 5;  // 32-row fragments with rows: 1..8
            nv = __builtin_amdgcn_readfirstlane((nfrag - wm + 1) >> 1);
            na = __builtin_amdgcn_readfirstlane(min(max(nfrag * 32 - wid * 64, 0) / RPL, LOADS));
        }
        const int brow0 = SWIGLU ? nt * 128 : nt * kTile;
        // row of A (tile-relative, or of x when gathering) that tile row r reads
        auto a_row = [&](int r) -> int {
            const int ar = min(row0 + r, a_end - 1);
            return p.src_map ? p.src_map[ar] / p.gk : ar - row0;
        };
        // B row (of the expert's matrix) that tile row r of B holds
        auto b_row = [&](int r) -> int {
            if (SWIGLU) {
                const int f = min(nt * 128 + (r & 127), p.n_out - 1);
                return r < 128 ? f : p.n_out + f;
            }
            return min(nt * kTile + out_col(r), p.n_out - 1);
        };
        // Per-lane load offsets from an opaque copy of the lane index, so the
        // compiler forms them per tile instead of holding per-lane constants
        // across the K loop.
        int sl = lane;
        __asm__ volatile("" : "+v"(sl));
        const int lrow = sl / CH, lslot = sl % CH;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int r = wid * 64 + i * RPL + lrow;  // tile row 0..255
            const int chunk = lslot ^ swz<1>(r);
            aoff[i] = (uint32_t)((size_t)a_row(r) * KB + chunk * 16);
            boff[i] = (uint32_t)((size_t)(b_row(r) - brow0) * KB + chunk * 16);
        }
        {
            const int r = wid * 64 + sl;  // tile row of this lane's scale words
            asoff = (uint32_t)(a_row(r) * KS);
            bsoff = (uint32_t)((b_row(r) - brow0) * KS);
        }
        acodes = p.src_map ? p.A : p.A + (size_t)row0 * KB;
        bcodes = p.B + ((size_t)e * p.b_rows + brow0) * KB;
        ascale = p.src_map ? p.As : p.As + (size_t)row0 * KS;
        bscale = p.Bs + ((size_t)e * p.b_rows + brow0) * KS;
        MX_SB;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            MX_LOAD_A(kb, 0, i);
            MX_LOAD_B(kb, 0, i);
        }
        // (no K split here: kb = 0, so stage kt's buffer is kt % 2)
        MX_LOAD_AS(0, 0);
        MX_LOAD_BS(0, 0);
        const int k1 = min(kb + 1, ke - 1);
#pragma unroll
        for (int i = 0; i < LOADS; ++i) MX_LOAD_A(k1, 1, i);
        if constexpr (G == 1) MX_LOAD_AS(k1, 1);
        MX_SB;
    };
    // The B half of the unit's second stage (into stage buffer 1).
    auto load_b_half = [&]() __attribute__((always_inline)) {
        if (!valid) return;
        const int k1 = min(kb + 1, ke - 1);
        MX_SB;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) MX_LOAD_B(k1, 1, i);
        if constexpr (G == 1) MX_LOAD_BS(k1, 1);
        MX_SB;
    };

    setup(unit);
    load_b_half();
    while (unit >= 0) {
        i32x8 fa0[4], fb0[4], fa1[4], fb1[4];
        constexpr int NSW = F4 ? 16 : 8;  // scale words of a stage a lane uses (shifted: ss)
        uint32_t sw[8], ss[NSW];
        uint2 sw2[8];  // E2M1: both words of each fragment row
        // the unit's first two stages landed everywhere; the previous unit's stores retired
        __asm__ volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        MX_SB;
        if (tid == 0) {  // publish the next unit, take a ticket for the one after
            const int nu = take(tick);
            s_unit = nu;
            tick = nu >= 0 ? ticket() : -1;
        }
        // The accumulators live in the accumulator registers for the whole
        // tile: empty asm statements with "a" constraints (at the zeroing and
        // once per stage) keep the register allocator from moving them
        // through VGPRs around the MFMAs that the fragment count may skip.
        f32x16 acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                f32x16 z;
#pragma unroll
                for (int q = 0; q < 16; ++q) z[q] = 0.f;
                __asm__ volatile("" : "=a"(acc[i][j]) : "0"(z));
            }
#define MX_PIN_ACC(I)                                                                                    \
    __asm__ volatile("" : "+a"(acc[I][0]), "+a"(acc[I][1]), "+a"(acc[I][2]), "+a"(acc[I][3]))
        MX_RD_A(fa0, 0u, 0, 0);
        MX_RD_A(fa0, 0u, 0, 1);
        MX_RD_A(fa0, 0u, 0, 2);
        MX_RD_A(fa0, 0u, 0, 3);
        MX_RD_B(fb0, 0u, 0, 0);
        MX_RD_B(fb0, 0u, 0, 1);
        MX_RD_B(fb0, 0u, 0, 2);
        MX_RD_B(fb0, 0u, 0, 3);
        MX_RD_S(sw, MX_SC_OFF(kb));
        MX_WAIT_F(fa0, fb0);
        MX_WAIT_W(sw);
// One stage KT in stage buffer ST (0 or 1); SCL (a literal): whether its
// second K step issues scale-word loads.  G = 1: those of stage kl, into the
// freed slot ST; G = 4 (every fourth stage): the next group of four stages,
// into the other slot.
#define MX_STAGE(KT, ST, SCL)                                                                            \
    {                                                                                                    \
        const int kt_ = (KT), st_ = (ST);                                                                \
        const uint32_t so = st_ ? STB : 0u, nso = st_ ? 0u : STB;                                        \
        const int kl = min(kt_ + 2, ke - 1); /* loads of stage kt+2 (past the end: the last stage) */   \
        const int sg = G == 1 ? kl : min(kt_ / G + 1, (ke - 1) / G);                                     \
        const int sslot = G == 1 ? st_ : ((kt_ / G) + 1) & 1;                                            \
        const uint32_t nsc = MX_SC_OFF(kt_ + 1);                                                         \
        MX_PIN_ACC(0); MX_PIN_ACC(1); MX_PIN_ACC(2); MX_PIN_ACC(3);                                      \
        MX_SB;                                                                                           \
        if constexpr (F4) {                                                                              \
            _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                              \
                ss[2 * i] = sw2[i].x >> (8 * half);                                                      \
                ss[2 * i + 1] = sw2[i].y >> (8 * half);                                                  \
            }                                                                                            \
        } else {                                                                                         \
            _Pragma("unroll") for (int i = 0; i < 8; ++i) ss[i] = sw[i] >> (8 * half);                   \
        }                                                                                                \
        MX_SB;                                                                                           \
        /* K step 0 on fa0/fb0; the fragments of K step 1 are read under the first 8 MFMAs */           \
        MX_STEP(fa0, fb0, ss, 0, 0, 0, (void)0, MX_RD_A(fa1, so, 1, 0))                                  \
        MX_STEP(fa0, fb0, ss, 0, 0, 1, (void)0, MX_RD_A(fa1, so, 1, 1))                                  \
        MX_STEP(fa0, fb0, ss, 0, 0, 2, (void)0, MX_RD_A(fa1, so, 1, 2))                                  \
        MX_STEP(fa0, fb0, ss, 0, 0, 3, (void)0, MX_RD_A(fa1, so, 1, 3))                                  \
        MX_STEP(fa0, fb0, ss, 0, 1, 0, (void)0, MX_RD_B(fb1, so, 1, 0))                                  \
        MX_STEP(fa0, fb0, ss, 0, 1, 1, (void)0, MX_RD_B(fb1, so, 1, 1))                                  \
        MX_STEP(fa0, fb0, ss, 0, 1, 2, (void)0, MX_RD_B(fb1, so, 1, 2))                                  \
        MX_STEP(fa0, fb0, ss, 0, 1, 3, (void)0, MX_RD_B(fb1, so, 1, 3))                                  \
        MX_STEP(fa0, fb0, ss, 0, 2, 0, (void)0, (void)0)                                                 \
        MX_STEP(fa0, fb0, ss, 0, 2, 1, (void)0, (void)0)                                                 \
        MX_STEP(fa0, fb0, ss, 0, 2, 2, (void)0, (void)0)                                                 \
        MX_STEP(fa0, fb0, ss, 0, 2, 3, (void)0, (void)0)                                                 \
        MX_STEP(fa0, fb0, ss, 0, 3, 0, (void)0, (void)0)                                                 \
        MX_STEP(fa0, fb0, ss, 0, 3, 1, (void)0, (void)0)                                                 \
        MX_STEP(fa0, fb0, ss, 0, 3, 2, (void)0, (void)0)                                                 \
        MX_STEP(fa0, fb0, ss, 0, 3, 3, (void)0, (void)0)                                                 \
        MX_WAIT_F(fa1, fb1);                                                                             \
        /* this wave has read all of stage kt; past the barrier the same holds */                       \
        /* for every wave, and buffer ST is free */                                                      \
        __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");                              \
        MX_SB;                                                                                           \
        /* K step 1 on fa1/fb1; the loads of stage kt+2 go into buffer ST, four */                      \
        /* of B first; then this wave's loads of stage kt+1 (and earlier scale */                       \
        /* words) have landed: only those four are younger, and vector memory */                        \
        /* operations complete in issue order; past a second barrier stage */                           \
        /* kt+1's first fragments and scale words are read */                                            \
        MX_STEP(fa1, fb1, ss, 1, 0, 0, MX_LOAD_B(kl, st_, 0), (void)0)                                   \
        MX_STEP(fa1, fb1, ss, 1, 0, 1, MX_LOAD_B(kl, st_, 1), (void)0)                                   \
        MX_STEP(fa1, fb1, ss, 1, 0, 2, MX_LOAD_B(kl, st_, 2), (void)0)                                   \
        MX_STEP(fa1, fb1, ss, 1, 0, 3, MX_LOAD_B(kl, st_, 3), (void)0)                                   \
        __asm__ volatile("s_waitcnt vmcnt(4)\n\ts_barrier" ::: "memory");                                \
        MX_SB;                                                                                           \
        MX_STEP(fa1, fb1, ss, 1, 1, 0, MX_LOAD_A_IF(kl, st_, 0), MX_RD_A(fa0, nso, 0, 0))                   \
        MX_STEP(fa1, fb1, ss, 1, 1, 1, MX_LOAD_A_IF(kl, st_, 1), MX_RD_A(fa0, nso, 0, 1))                   \
        MX_STEP(fa1, fb1, ss, 1, 1, 2, MX_LOAD_A_IF(kl, st_, 2), MX_RD_A(fa0, nso, 0, 2))                   \
        MX_STEP(fa1, fb1, ss, 1, 1, 3, MX_LOAD_A_IF(kl, st_, 3), MX_RD_A(fa0, nso, 0, 3))                   \
        MX_STEP(fa1, fb1, ss, 1, 2, 0, MX_LOAD_A_IF(kl, st_, 4); if (SCL) MX_LOAD_AS(sg, sslot), MX_RD_B(fb0, nso, 0, 0)) \
        MX_STEP(fa1, fb1, ss, 1, 2, 1, MX_LOAD_A_IF(kl, st_, 5), MX_RD_B(fb0, nso, 0, 1))                   \
        MX_STEP(fa1, fb1, ss, 1, 2, 2, MX_LOAD_A_IF(kl, st_, 6), MX_RD_B(fb0, nso, 0, 2))                   \
        MX_STEP(fa1, fb1, ss, 1, 2, 3, MX_LOAD_A_IF(kl, st_, 7), MX_RD_B(fb0, nso, 0, 3))                   \
        MX_STEP(fa1, fb1, ss, 1, 3, 0, MX_LOAD_B(kl, st_, 4), MX_RD_S(sw, nsc))                          \
        MX_STEP(fa1, fb1, ss, 1, 3, 1, MX_LOAD_B(kl, st_, 5), (void)0)                                   \
        MX_STEP(fa1, fb1, ss, 1, 3, 2, MX_LOAD_B(kl, st_, 6), (void)0)                                   \
        MX_STEP(fa1, fb1, ss, 1, 3, 3, MX_LOAD_B(kl, st_, 7); if (SCL) MX_LOAD_BS(sg, sslot), (void)0)   \
        /* the next stage's first fragments and scale words landed (no LDS read */                      \
        /* is in flight when the loop ends) */                                                           \
        MX_WAIT_F(fa0, fb0);                                                                             \
        MX_WAIT_W(sw);                                                                                   \
    }
        if constexpr (G == 1) {
            for (int kt = kb; kt < ke; ++kt) MX_STAGE(kt, (kt - kb) & 1, 1)
        } else if constexpr (G == 2) {
            // stages in twos (K is a multiple of 2 stages, kb = 0)
            for (int kt = kb; kt < ke; kt += 2) {
                MX_STAGE(kt, 0, 1)
                MX_STAGE(kt + 1, 1, 0)
            }
        } else {
            // stages in fours (K is a multiple of 4 stages, kb = 0): the scale
            // group loads sit in the first stage of each four, with no branch
            for (int kt = kb; kt < ke; kt += 4) {
                MX_STAGE(kt, 0, 1)
                MX_STAGE(kt + 1, 1, 0)
                MX_STAGE(kt + 2, 0, 0)
                MX_STAGE(kt + 3, 1, 0)
            }
        }
#undef MX_STAGE
#undef MX_PIN_ACC
        MX_SB;
#undef MX_LOAD_A
#undef MX_LOAD_A_IF
#undef MX_LOAD_B
#undef MX_LOAD_SC
#undef MX_LOAD_AS
#undef MX_LOAD_BS
#undef MX_SC_OFF
#undef MX_RD_A
#undef MX_RD_B
#undef MX_RD_S
#undef MX_WAIT_F
#undef MX_WAIT_W
#undef MX_MFMA
#undef MX_STEP
        // every wave has read its last stage; the next unit (published by
        // thread 0 before this unit's K loop) gets its first loads now
        __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        const int next_unit = s_unit;
        const int e_row0 = row0, e_row_end = row_end, e_a_end = a_end, e_nt = nt;
        const bool e_valid = valid;
        // routing weights of this wave's 128 rows, two per lane (its rows
        // 2 lane and 2 lane + 1; its row i is tile row 32 (2 (i / 32) + wm) +
        // i % 32), loaded and waited for before setup issues the next unit's
        // loads
        float rwa = 1.f, rwb = 1.f;
        if constexpr ((EP & 1) != 0) {
            if (e_valid) {
                const float* const rwp = p.row_w + e_row0 + 32 * (2 * (lane >> 4) + wm) + ((2 * lane) & 31);
                rwa = rwp[0];
                rwb = rwp[1];
            }
            __asm__ volatile("" : "+v"(rwa), "+v"(rwb));
        }
        if (next_unit >= 0) setup(next_unit);
        if (e_valid) {
            int rbase = e_row0, ln = lane;
            __asm__ volatile("" : "+v"(rbase), "+v"(ln));
            const int rlim = e_row_end - rbase;  // rows of the tile that exist
            const int alim = e_a_end - rbase;    // rows of the tile that are not padding (gather)
            if (SWIGLU) {
                // this wave's LDS tile (32 x 33 floats) in its own B rows of
                // stage buffer 1; the loop's last loads (repeats of the last
                // stage, possibly into these rows) must have landed first:
                // they precede the 27 (G = 4: 26) loads of setup (if it issued any)
                if (next_unit >= 0 && valid) {
                    if constexpr (G == 1) __asm__ volatile("s_waitcnt vmcnt(27)" ::: "memory");
                    else __asm__ volatile("s_waitcnt vmcnt(26)" ::: "memory");
                } else {
                    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
                }
                float* const wb = (float*)(lds + STB + OPB + wid * 64 * BKB);
                const int rr = ln >> 1, cc = (ln & 1) * 16;
#define MX_EPI_SW(MI, NI)                                                                                \
    {                                                                                                    \
        float hv[16];                                                                                    \
        _Pragma("unroll") for (int q = 0; q < 16; ++q)                                                   \
            hv[q] = (EP & 2) != 0 ? silu(fminf(agpr_read(acc[MI][NI][q]), p.lim)) *                      \
                                        fminf(fmaxf(agpr_read(acc[MI][(NI) + 2][q]), -p.lim), p.lim)     \
                                  : silu(agpr_read(acc[MI][NI][q])) * agpr_read(acc[MI][(NI) + 2][q]);   \
        GE_STAGE_TILE(wb, hv)                                                                            \
        __builtin_amdgcn_s_waitcnt(0xC07F);                                                              \
        float v[16];                                                                                     \
        float amax = 0.f;                                                                                \
        const bool pad = (2 * (MI) + wm) * 32 + rr >= alim; /* gather: padding rows are zeros */        \
        float rw = 1.f;                                                                                  \
        if constexpr ((EP & 1) != 0) {                                                                              \
            const float wa_ = __shfl(rwa, ((MI) * 32 + rr) >> 1, 64);                                    \
            const float wb_ = __shfl(rwb, ((MI) * 32 + rr) >> 1, 64);                                    \
            rw = (rr & 1) ? wb_ : wa_;                                                                   \
        }                                                                                                \
        _Pragma("unroll") for (int j = 0; j < 16; ++j) {                                                 \
            v[j] = pad ? 0.f : wb[rr * 33 + cc + j] * rw;                                                \
            amax = fmaxf(amax, fabsf(v[j]));                                                             \
        }                                                                                                \
        __builtin_amdgcn_s_waitcnt(0xC07F);                                                              \
        amax = fmaxf(amax, __shfl_xor(amax, 1, 64));                                                     \
        const int r = (2 * (MI) + wm) * 32 + rr;                                                         \
        const int f = e_nt * 128 + wn * 64 + (NI) * 32 + cc;                                             \
        if (r < rlim && f < p.n_out) {                                                                   \
            const size_t row = (size_t)(rbase + r);                                                      \
            int se;                                                                                      \
            if constexpr (F4) {                                                                          \
                se = mx4_shared_exp(amax);                                                               \
                uint32_t w2[2] = {0u, 0u};                                                               \
                _Pragma("unroll") for (int j = 0; j < 16; ++j)                                           \
                    w2[j >> 3] |= (uint32_t)e2m1_rne(ldexpf(v[j], -se)) << (4 * (j & 7));                \
                *(uint2*)(p.C + row * (p.n_out / 2) + f / 2) = make_uint2(w2[0], w2[1]);                 \
            } else {                                                                                     \
                se = mx_shared_exp(amax);                                                                \
                uint32_t w4[4];                                                                          \
                _Pragma("unroll") for (int j = 0; j < 4; ++j)                                            \
                    w4[j] = (uint32_t)e4m3_rne(ldexpf(v[4 * j], -se)) |                                  \
                            ((uint32_t)e4m3_rne(ldexpf(v[4 * j + 1], -se)) << 8) |                       \
                            ((uint32_t)e4m3_rne(ldexpf(v[4 * j + 2], -se)) << 16) |                      \
                            ((uint32_t)e4m3_rne(ldexpf(v[4 * j + 3], -se)) << 24);                       \
                *(uint4*)(p.C + row * p.n_out + f) = make_uint4(w4[0], w4[1], w4[2], w4[3]);             \
            }                                                                                            \
            if ((ln & 1) == 0) p.Cs[row * (p.n_out / 32) + f / 32] = (uint8_t)(se + 127);                \
        }                                                                                                \
        if (p.stash) {                                                                                   \
            _Pragma("unroll") for (int gu = 0; gu < 2; ++gu) {                                           \
                float tv[16];                                                                            \
                _Pragma("unroll") for (int q = 0; q < 16; ++q)                                           \
                    tv[q] = agpr_read(acc[MI][(NI) + 2 * gu][q]);                                        \
                GE_STAGE_TILE(wb, tv)                                                                    \
                __builtin_amdgcn_s_waitcnt(0xC07F);                                                      \
                float sv[16];                                                                            \
                _Pragma("unroll") for (int j = 0; j < 16; ++j) sv[j] = wb[rr * 33 + cc + j];             \
                __builtin_amdgcn_s_waitcnt(0xC07F);                                                      \
                if (r < rlim && f < p.n_out) {                                                           \
                    uint4* const d = (uint4*)(p.stash + (size_t)(rbase + r) * 2 * p.n_out + gu * p.n_out + f); \
                    d[0] = GE_PACK8(sv, 0);                                                              \
                    d[1] = GE_PACK8(sv, 8);                                                              \
                }                                                                                        \
            }                                                                                            \
        }                                                                                                \
    }                                                                                                    \
    __builtin_amdgcn_sched_barrier(0);
                MX_EPI_SW(0, 0) MX_EPI_SW(0, 1) MX_EPI_SW(1, 0) MX_EPI_SW(1, 1)
                MX_EPI_SW(2, 0) MX_EPI_SW(2, 1) MX_EPI_SW(3, 0) MX_EPI_SW(3, 1)
#undef MX_EPI_SW
                // this wave's reads of its LDS tile are done before its loads refill those rows
                __builtin_amdgcn_s_waitcnt(0xC07F);
            } else {
                const int lc = ln & 31, lr = 4 * (ln >> 5);
                uint16_t* const cbase = p.Cb + (size_t)rbase * p.n_out;
                const int n = e_nt * kTile + wn * 128 + 4 * lc;  // this lane's columns n .. n + 3
                // Yp goes out with nontemporal stores (st_nt), ~1 % faster here;
                // the gate/up epilogue above keeps plain stores for h, its scale
                // bytes and the stash, which measured 2-6 % faster than
                // nontemporal ones.
#define MX_EPI_DN(MI)                                                                                    \
    {                                                                                                    \
        const int rb0 = (2 * (MI) + wm) * 32;                                                            \
        uint2 w[16];                                                                                     \
        float rw[16];                                                                                    \
        if constexpr ((EP & 1) != 0) {                                                                              \
            _Pragma("unroll") for (int q = 0; q < 16; ++q)                                               \
                rw[q] = __shfl((q & 1) ? rwb : rwa, ((MI) * 32 + lr + 8 * (q >> 2) + (q & 3)) >> 1, 64); \
        } else {                                                                                         \
            _Pragma("unroll") for (int q = 0; q < 16; ++q) rw[q] = 1.f;                                  \
        }                                                                                                \
        _Pragma("unroll") for (int q = 0; q < 16; ++q)                                                   \
            w[q] = make_uint2(pack_bf16x2(agpr_read(acc[MI][0][q]) * rw[q], agpr_read(acc[MI][1][q]) * rw[q]), \
                              pack_bf16x2(agpr_read(acc[MI][2][q]) * rw[q], agpr_read(acc[MI][3][q]) * rw[q])); \
        if (n < p.n_out) {                                                                               \
            uint16_t* const dst = cbase + (size_t)(rb0 + lr) * p.n_out + n;                              \
            if (rb0 + 32 <= rlim) {                                                                      \
                _Pragma("unroll") for (int q = 0; q < 16; ++q)                                           \
                    st_nt((uint2*)(dst + (size_t)(8 * (q >> 2) + (q & 3)) * p.n_out), w[q]);             \
            } else {                                                                                     \
                _Pragma("unroll") for (int q = 0; q < 16; ++q)                                           \
                    if (rb0 + lr + 8 * (q >> 2) + (q & 3) < rlim)                                        \
                        st_nt((uint2*)(dst + (size_t)(8 * (q >> 2) + (q & 3)) * p.n_out), w[q]);         \
            }                                                                                            \
        }                                                                                                \
    }                                                                                                    \
    __builtin_amdgcn_sched_barrier(0);
                MX_EPI_DN(0) MX_EPI_DN(1) MX_EPI_DN(2) MX_EPI_DN(3)
#undef MX_EPI_DN
            }
        }  // valid
        if (next_unit >= 0) load_b_half();
        unit = next_unit;
    }
    // no direct-to-LDS load may still be in flight when the wave ends
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
#undef MX_SB
}

}  // namespace gemm
}  // namespace moe
