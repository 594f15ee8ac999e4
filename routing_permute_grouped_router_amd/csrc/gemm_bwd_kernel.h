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
// accumulators), two LDS stages of 64 KiB filled straight from global memory
// (global_load_lds, 16-byte pieces; the next stage is in flight while the
// current one feeds the matrix cores).  A K-contiguous operand (the rows of a
// DGRAD) is kept as in the forward kernel: 128-byte rows of 64 K values, the
// 16-byte chunks XOR-permuted by (row & 7).  A strided operand (the weights of
// a DGRAD; both operands of a WGRAD) is kept as it lies in memory: 64 K rows of
// 256 columns (512 bytes each), 16-byte chunk c of K row k stored at chunk
// position c ^ 4 (k & 3), and its MFMA fragments are read with the CDNA4 LDS
// transpose read ds_read_b64_tr_b16.  Measured lane rule of that instruction:
// within each group of 16 lanes, lane i receives element i % 4 of the four
// 16-bit values addressed by lanes i / 4, i / 4 + 4, i / 4 + 8, i / 4 + 12.
// Lane a of a group therefore addresses K row kb + a / 4, columns c + 4 (a % 4)
// and receives column c + a at K rows kb .. kb + 3; two such reads give the
// eight K values of one MFMA operand lane.  The 4 (k & 3) chunk permutation
// puts the four K rows of one read in different LDS banks.
// Rows past a WGRAD unit's end load a clamped valid row and the A copy of
// those rows is overwritten with zeros before use; rows and columns past a
// DGRAD's output are never stored.
#pragma once

#include "gemm_bf16_kernel.h"

namespace moe {
namespace gemm {

// kDgradDswigluClamp: kDgradDswiglu for a forward with the SwiGLU clamp (a
// separate instance, so the plain one carries no clamp work per element).
enum BwdMode { kDgrad = 0, kDgradDswiglu = 1, kWgrad = 2, kDgradDswigluClamp = 3 };

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
    // Tile counters, one per XCD, zero at launch: the blocks of an XCD take
    // their next tile from the XCD's list with an atomic increment.
    int* sched;
    // kDgradDswigluClamp: the forward's SwiGLU clamp limit; the
    // gradient of a clamped gate or up value is 0, values on a bound pass
    float lim;
};

constexpr int kMaxUnits = 2048;  // weight-gradient units dealt by size (beyond: by index)

// Hand the tile index that thread 0 fetched (nxt) to the whole block.
__device__ __forceinline__ int bwd_next_tile(int* s_next, int& sb, int nxt) {
    if (threadIdx.x == 0) s_next[sb ^ 1] = nxt;
    __syncthreads();
    sb ^= 1;
    return s_next[sb];
}

// Byte offset, within a [64][256] strided stage region, that lane `lane`
// addresses for the 32-column block starting at colbase (K base 0).
__device__ __forceinline__ uint32_t tr_lane_off(int colbase, int lane) {
    const int a = lane & 15, g = (lane >> 4) & 1;
    const int col = colbase + 16 * g + 4 * (a & 3);
    const int krow = a >> 2;  // K row within a group of four (K base is a multiple of 4)
    return (uint32_t)(krow * 512 + (((col >> 3) ^ (krow << 2)) << 4) + (col & 7) * 2);
}

// LDS reads issued as inline asm: the compiler then does not order them
// behind the direct-to-LDS loads still in flight into the other stage (it
// cannot tell the two stages apart); waits are explicit (bwd_wait).
__device__ __forceinline__ uint4 bwd_ds_read16(uint32_t addr) {
    uint4 v;
    __asm__ volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr) : "memory");
    return v;
}
__device__ __forceinline__ uint2 bwd_ds_read_tr(uint32_t addr) {
    uint2 v;
    __asm__ volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(addr) : "memory");
    return v;
}
// eight K values of one operand lane from two transpose reads, 2048 bytes apart
__device__ __forceinline__ bf16x8 bwd_tr_frag(uint32_t addr) {
    const uint2 lo = bwd_ds_read_tr(addr), hi = bwd_ds_read_tr(addr + 4 * 512);
    return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}
#define BWD_WAIT(FA, FB)                                                                                  \
    __asm__ volatile("s_waitcnt lgkmcnt(0)"                                                               \
                     : "+v"(FA[0]), "+v"(FA[1]), "+v"(FA[2]), "+v"(FA[3]), "+v"(FB[0]), "+v"(FB[1]),     \
                       "+v"(FB[2]), "+v"(FB[3])::"memory")

template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_bwd(BwdArgs p) {
    constexpr int BK = 64;
    constexpr bool WG = MODE == kWgrad;
    constexpr bool DSW = MODE == kDgradDswiglu || MODE == kDgradDswigluClamp;  // SwiGLU backward epilogue
    constexpr int OPB = kTile * BK * 2;  // bytes of one operand in one stage
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2][2][OPB];
    __shared__ int32_t pre[kMaxExperts + 1];
    __shared__ int32_t spre[WG ? kMaxExperts + 1 : 1];
    __shared__ int scan_tmp[kThreads / 64];

    const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wid >> 1, wn = wid & 1, half = lane >> 5;
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
    const int xcd = blockIdx.x % kXcds;
    // Row-indexed GEMMs: every tile costs the same; each XCD owns a
    // contiguous range of the tile sequence.  Weight gradients: units differ
    // in rows, so they are ranked by rows (longest first) and dealt to the
    // XCDs in snake order (ranks 0..7 to XCDs 0..7, ranks 8..15 to XCDs
    // 7..0, ...), which evens out the XCDs' loads; an XCD lists its units in
    // rank order.  In both cases the blocks of an XCD take tiles from the
    // XCD's list through its counter, so a block that finishes early takes
    // the next tile.
    __shared__ int32_t ukey[WG ? kMaxUnits : 1];
    __shared__ int32_t uorder[WG ? kMaxUnits / kXcds + 1 : 1];
    __shared__ int s_next[2];
    int t_begin, t_end, nj = 0;
    const int mn = m_tiles * n_tiles;
    const bool dealt = WG && total / max(mn, 1) <= kMaxUnits;
    if (WG) {
        const int units = total / mn;
        if (dealt) {
            for (int u = tid; u < units; u += kThreads) {
                const int e = find_expert(pre, p.E, u);
                const int r_begin = max(0, p.offsets[e]), r_end = min(p.offsets[e + 1], p.rows);
                const int kb = min(r_begin + (u - pre[e]) * p.S, r_end);
                ukey[u] = min(kb + p.S, r_end) - kb;
            }
            __syncthreads();
            for (int u = tid; u < units; u += kThreads) {
                const int ku = ukey[u];
                int rank = 0;
                for (int i = 0; i < units; ++i) {
                    const int ki = ukey[i];
                    rank += ki > ku || (ki == ku && i < u);
                }
                const int round = rank / kXcds, pos = rank % kXcds;
                if (((round & 1) ? kXcds - 1 - pos : pos) == xcd) uorder[round] = u;
            }
            const int full = units / kXcds, rest = units % kXcds;
            nj = full + (((full & 1) ? kXcds - 1 - xcd : xcd) < rest ? 1 : 0);
        } else {
            nj = units > xcd ? (units - xcd + kXcds - 1) / kXcds : 0;
        }
        t_begin = 0;
        t_end = nj * mn;
    } else {
        t_begin = (int)((int64_t)total * xcd / kXcds);
        t_end = (int)((int64_t)total * (xcd + 1) / kXcds);
    }
    int sb = 0, nxt = 0;
    if (tid == 0) s_next[0] = atomicAdd(p.sched + xcd, 1);
    __syncthreads();
    const int t_first = t_begin + s_next[0];

    // fragment addressing: K-contiguous A rows (DGRAD) and strided blocks
    int arow[4];
    uint32_t a_tr[4], b_tr[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        arow[mi] = wm * 128 + mi * 32 + (lane & 31);
        a_tr[mi] = tr_lane_off(wm * 128 + mi * 32, lane);
    }
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) b_tr[ni] = tr_lane_off(wn * 128 + ni * 32, lane);
    // loaders: K-contiguous rows r = wid*64 + 8i + lane/8, chunk lane%8 (permuted by r & 7);
    // strided K rows kr = 16 wid + 2i + lane/32, chunk position lane%32 (holds chunk pos ^ 4 (kr & 3))
    const int c_lrow = lane >> 3, c_slot = lane & 7;
    const int s_kr = lane >> 5, s_pos = lane & 31;

    for (int t = t_first; t < t_end; t = t_begin + bwd_next_tile(s_next, sb, nxt)) {
        if (tid == 0) nxt = atomicAdd(p.sched + xcd, 1);  // the tile after this one; read at its end
        int e, m0, n0, k_begin, k_end, row0 = 0, row_end = 0;
        float* cw = nullptr;
        if (WG) {
            const int jl = t / mn;
            const int rem = t - jl * mn;
            const int u = dealt ? uorder[jl] : xcd + kXcds * jl;
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
        // the tile's coordinates are uniform: the load bases live in SGPRs
        e = __builtin_amdgcn_readfirstlane(e);
        m0 = __builtin_amdgcn_readfirstlane(m0);
        n0 = __builtin_amdgcn_readfirstlane(n0);
        k_begin = __builtin_amdgcn_readfirstlane(k_begin);
        k_end = __builtin_amdgcn_readfirstlane(k_end);
        row0 = __builtin_amdgcn_readfirstlane(row0);
        row_end = __builtin_amdgcn_readfirstlane(row_end);
        const int nk = k_end > k_begin ? (k_end - k_begin + BK - 1) / BK : 0;

        // per-lane byte offsets of the 8 loads of each operand, for K step 0
        //   A: DGRAD rows of p.A [rows][K]; WGRAD K rows of p.A [rows][M] (columns m0..)
        //   B: DGRAD K rows of B_e [K][N] (columns n0..); WGRAD K rows of p.B [rows][N]
        const char* abase;
        const char* bbase;
        size_t a_kstep, b_kstep;  // bytes per K step of 64
        uint32_t aoff[8], boff[8];
        const int ncols_b = p.N;
        if (WG) {
            abase = (const char*)(p.A + (size_t)k_begin * p.M);
            bbase = (const char*)(p.B + (size_t)k_begin * p.N);
            a_kstep = (size_t)BK * p.M * 2;
            b_kstep = (size_t)BK * p.N * 2;
        } else {
            abase = (const char*)(p.A + (size_t)row0 * p.K);
            bbase = (const char*)(p.B + (size_t)e * p.K * p.N);
            a_kstep = BK * 2;
            b_kstep = (size_t)BK * p.N * 2;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int kr = 16 * wid + 2 * i + s_kr;                   // strided: K row within the stage
            const int sch = s_pos ^ ((kr & 3) << 2);                   // global chunk this lane fetches
            const int ncol = min(n0 + 8 * sch, ncols_b - 8);           // clamp to a valid chunk
            if (WG) {
                const int mcol = min(m0 + 8 * sch, p.M - 8);
                aoff[i] = (uint32_t)(((size_t)kr * p.M + mcol) * 2);
                boff[i] = (uint32_t)(((size_t)kr * p.N + ncol) * 2);
            } else {
                const int r = wid * 64 + 8 * i + c_lrow;                // K-contiguous: tile row
                const int ar = min(row0 + r, row_end - 1);
                aoff[i] = (uint32_t)(((size_t)(ar - row0) * p.K + 8 * (c_slot ^ (r & 7))) * 2);
                boff[i] = (uint32_t)(((size_t)kr * p.N + ncol) * 2);
            }
        }
        // WGRAD: K rows past the unit's end load row k_end-1 instead (zeroed in A below)
        int a_rowcap = 0;
        if (WG) a_rowcap = k_end - k_begin - 1;

        f32x16 acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

        // Direct-to-LDS loads (dma_lds16: uniform M0 and base, 32-bit lane
        // offsets).  Stage kt of an operand starts at base + kt * kstep.
        // A WGRAD unit's last stage may run past its rows: there each lane
        // clamps its K row to the unit's last row (the only stage that needs
        // per-lane arithmetic), and the A copy of those rows is zeroed once
        // they have landed (this wave's own rows).
        const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void*)&lds[0][0][0];
        const uint32_t a_dst = __builtin_amdgcn_readfirstlane(lds_base + (uint32_t)(WG ? 16 * wid * 512 : wid * 64 * 128));
        const uint32_t b_dst = __builtin_amdgcn_readfirstlane(lds_base + OPB + (uint32_t)(16 * wid * 512));
        // stage kt reaches past the WGRAD unit's rows
#define GB_TAIL(kt) (WG && (kt) * BK + BK - 1 > a_rowcap)
#define GB_LOAD_A(kt, st, i)                                                                              \
    {                                                                                                     \
        uint32_t o_ = aoff[i];                                                                            \
        if (GB_TAIL(kt)) {                                                                                \
            const int kr_ = (kt) * BK + 16 * wid + 2 * (i) + s_kr;                                        \
            if (kr_ > a_rowcap) o_ -= (uint32_t)(kr_ - a_rowcap) * (uint32_t)p.M * 2u;                    \
        }                                                                                                 \
        dma_lds16(a_dst + (uint32_t)(st) * 2 * OPB + (i) * (WG ? 2 * 512 : 8 * 128), o_,                  \
                  abase + (size_t)(kt) * a_kstep);                                                        \
    }
#define GB_LOAD_B(kt, st, i)                                                                              \
    {                                                                                                     \
        uint32_t o_ = boff[i];                                                                            \
        if (GB_TAIL(kt)) {                                                                                \
            const int kr_ = (kt) * BK + 16 * wid + 2 * (i) + s_kr;                                        \
            if (kr_ > a_rowcap) o_ -= (uint32_t)(kr_ - a_rowcap) * (uint32_t)p.N * 2u;                    \
        }                                                                                                 \
        dma_lds16(b_dst + (uint32_t)(st) * 2 * OPB + (i) * 2 * 512, o_, bbase + (size_t)(kt) * b_kstep);  \
    }
        // WGRAD tail: zero the A copy of K rows past the unit's end (this wave's
        // own rows; every load of this wave has landed)
#define GB_ZERO_TAIL(kt, st)                                                                              \
    if (GB_TAIL(kt)) {                                                                                    \
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");                                             \
        _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                                   \
            const int kr = 16 * wid + 2 * i + s_kr;                                                       \
            if ((kt) * BK + kr > a_rowcap) *(uint4*)&lds[st][0][kr * 512 + s_pos * 16] = make_uint4(0, 0, 0, 0); \
        }                                                                                                 \
    }
        // fragment reads of K sub-step kk of the stage in buffer st: A
        // fragment mi (one 16-byte read, or two transpose reads for a strided
        // A), B fragment ni (two transpose reads)
#define GB_RD_A(FA, st, kk, mi)                                                                           \
    FA[mi] = WG ? bwd_tr_frag(lds_base + (st) * 2 * OPB + a_tr[mi] + (16 * (kk) + 8 * half) * 512)        \
                : __builtin_bit_cast(bf16x8, bwd_ds_read16(lds_base + (st) * 2 * OPB + arow[mi] * 128 +   \
                                                           ((((kk) * 2 + half) ^ (arow[mi] & 7)) << 4)))
#define GB_RD_B(FB, st, kk, ni) FB[ni] = bwd_tr_frag(lds_base + (st) * 2 * OPB + OPB + b_tr[ni] + (16 * (kk) + 8 * half) * 512)
#define GB_MFMA(FA, FB, mi, ni) acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(FA[mi], FB[ni], acc[mi][ni], 0, 0, 0)
#define GB_SB __builtin_amdgcn_sched_barrier(0)
#define GB_STEP(FA, FB, mi, ni, PRE, RD)                                                                  \
    PRE;                                                                                                  \
    GB_MFMA(FA, FB, mi, ni);                                                                              \
    RD;                                                                                                   \
    GB_SB;
        // One K sub-step: 16 MFMAs on FA/FB; the 8 fragment reads of sub-step
        // KK (buffer ST) into GA/GB follow the first 8 of them, and L0..L7 (loads
        // of a later stage, or nothing) precede every other MFMA: one 1 KiB
        // load per two MFMAs per wave is what the CU's address unit sustains.
#define GB_SUBSTEP_X(FA, FB, GA, GB, ST, KK, L0, L1, L2, L3, L4, L5, L6, L7)                              \
    BWD_WAIT(FA, FB);                                                                                     \
    GB_SB;                                                                                                \
    GB_STEP(FA, FB, 0, 0, L0, GB_RD_A(GA, ST, KK, 0))                                                     \
    GB_STEP(FA, FB, 0, 1, (void)0, GB_RD_A(GA, ST, KK, 1))                                                \
    GB_STEP(FA, FB, 0, 2, L1, GB_RD_A(GA, ST, KK, 2))                                                     \
    GB_STEP(FA, FB, 0, 3, (void)0, GB_RD_A(GA, ST, KK, 3))                                                \
    GB_STEP(FA, FB, 1, 0, L2, GB_RD_B(GB, ST, KK, 0))                                                     \
    GB_STEP(FA, FB, 1, 1, (void)0, GB_RD_B(GB, ST, KK, 1))                                                \
    GB_STEP(FA, FB, 1, 2, L3, GB_RD_B(GB, ST, KK, 2))                                                     \
    GB_STEP(FA, FB, 1, 3, (void)0, GB_RD_B(GB, ST, KK, 3))                                                \
    GB_STEP(FA, FB, 2, 0, L4, (void)0)                                                                    \
    GB_STEP(FA, FB, 2, 1, (void)0, (void)0)                                                               \
    GB_STEP(FA, FB, 2, 2, L5, (void)0)                                                                    \
    GB_STEP(FA, FB, 2, 3, (void)0, (void)0)                                                               \
    GB_STEP(FA, FB, 3, 0, L6, (void)0)                                                                    \
    GB_STEP(FA, FB, 3, 1, (void)0, (void)0)                                                               \
    GB_STEP(FA, FB, 3, 2, L7, (void)0)                                                                    \
    GB_STEP(FA, FB, 3, 3, (void)0, (void)0)
#define GB_N_ (void)0
#define GB_SUBSTEP_NR(FA, FB)                                                                             \
    BWD_WAIT(FA, FB);                                                                                     \
    GB_SB;                                                                                                \
    GB_STEP(FA, FB, 0, 0, (void)0, (void)0) GB_STEP(FA, FB, 0, 1, (void)0, (void)0)                       \
    GB_STEP(FA, FB, 0, 2, (void)0, (void)0) GB_STEP(FA, FB, 0, 3, (void)0, (void)0)                       \
    GB_STEP(FA, FB, 1, 0, (void)0, (void)0) GB_STEP(FA, FB, 1, 1, (void)0, (void)0)                       \
    GB_STEP(FA, FB, 1, 2, (void)0, (void)0) GB_STEP(FA, FB, 1, 3, (void)0, (void)0)                       \
    GB_STEP(FA, FB, 2, 0, (void)0, (void)0) GB_STEP(FA, FB, 2, 1, (void)0, (void)0)                       \
    GB_STEP(FA, FB, 2, 2, (void)0, (void)0) GB_STEP(FA, FB, 2, 3, (void)0, (void)0)                       \
    GB_STEP(FA, FB, 3, 0, (void)0, (void)0) GB_STEP(FA, FB, 3, 1, (void)0, (void)0)                       \
    GB_STEP(FA, FB, 3, 2, (void)0, (void)0) GB_STEP(FA, FB, 3, 3, (void)0, (void)0)
#define GB_SUBSTEP(FA, FB, GA, GB, ST, KK)                                                                \
    GB_SUBSTEP_X(FA, FB, GA, GB, ST, KK, GB_N_, GB_N_, GB_N_, GB_N_, GB_N_, GB_N_, GB_N_, GB_N_)
#define GB_SUBSTEP_LA(FA, FB, GA, GB, ST, KK, LKT, LST)                                                   \
    GB_SUBSTEP_X(FA, FB, GA, GB, ST, KK, GB_LOAD_A(LKT, LST, 0), GB_LOAD_A(LKT, LST, 1), GB_LOAD_A(LKT, LST, 2), \
                 GB_LOAD_A(LKT, LST, 3), GB_LOAD_A(LKT, LST, 4), GB_LOAD_A(LKT, LST, 5), GB_LOAD_A(LKT, LST, 6), \
                 GB_LOAD_A(LKT, LST, 7))
#define GB_SUBSTEP_LB(FA, FB, GA, GB, ST, KK, LKT, LST)                                                   \
    GB_SUBSTEP_X(FA, FB, GA, GB, ST, KK, GB_LOAD_B(LKT, LST, 0), GB_LOAD_B(LKT, LST, 1), GB_LOAD_B(LKT, LST, 2), \
                 GB_LOAD_B(LKT, LST, 3), GB_LOAD_B(LKT, LST, 4), GB_LOAD_B(LKT, LST, 5), GB_LOAD_B(LKT, LST, 6), \
                 GB_LOAD_B(LKT, LST, 7))

        // Two LDS stages, software-pipelined as in the forward kernel: the
        // barrier of stage kt sits before its last sub-step (stage kt read by
        // every wave, stage kt+1 landed); after it the A half of stage kt+2
        // goes into the freed buffer under the last sub-step's MFMAs and the B
        // half under the first sub-step of stage kt+1, while the fragments of
        // the next sub-step are read under the MFMAs of the current one.
        // Loads past the last stage repeat it into the free buffer.
        bf16x8 f0a[4], f0b[4], f1a[4], f1b[4];
        if (nk > 0) {
            __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");  // previous tile's stores retired
            GB_SB;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                GB_LOAD_A(0, 0, i);
                GB_LOAD_B(0, 0, i);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) GB_LOAD_A(min(1, nk - 1), 1, i);
            __asm__ volatile("s_waitcnt vmcnt(8)" ::: "memory");  // stage 0 landed (this wave)
            GB_ZERO_TAIL(0, 0);
            __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            GB_SB;
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) GB_RD_A(f0a, 0, 0, mi);
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) GB_RD_B(f0b, 0, 0, ni);
        }
        for (int kt = 0; kt < nk; ++kt) {
            const int st = kt & 1;
            GB_SB;
            GB_SUBSTEP_LB(f0a, f0b, f1a, f1b, st, 1, min(kt + 1, nk - 1), st ^ 1)
            GB_SUBSTEP(f1a, f1b, f0a, f0b, st, 2)
            GB_SUBSTEP(f0a, f0b, f1a, f1b, st, 3)
            if (kt + 1 < nk) GB_ZERO_TAIL(kt + 1, st ^ 1);
            // this wave read all of stage kt and its loads of stage kt+1
            // landed; past the barrier, the same holds for every wave
            __asm__ volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
            GB_SB;
            GB_SUBSTEP_LA(f1a, f1b, f0a, f0b, st ^ 1, 0, min(kt + 2, nk - 1), st)
            // wait for the next stage's first fragments here (they had 8 MFMAs
            // to land), so no LDS read is in flight when the loop ends
            BWD_WAIT(f0a, f0b);
        }
        GB_SB;
#undef GB_TAIL
#undef GB_LOAD_A
#undef GB_LOAD_B
#undef GB_ZERO_TAIL
#undef GB_RD_A
#undef GB_RD_B
#undef GB_MFMA
#undef GB_SB
#undef GB_STEP
#undef GB_SUBSTEP_X
#undef GB_N_
#undef GB_SUBSTEP
#undef GB_SUBSTEP_LA
#undef GB_SUBSTEP_LB
#undef GB_SUBSTEP_NR
        // Weight gradients (float32) are stored straight from the
        // accumulators: lane l holds column l % 32 of each fragment, so one
        // 4-byte store per row and fragment writes two whole 128-byte rows
        // (lanes 0..31 and 32..63, four rows apart) -- the same bytes per
        // instruction as the LDS-staged form below would give, without its
        // LDS round trip.  Every output store of these kernels is
        // nontemporal (st_nt).
        // The dgrad epilogues go through LDS, so that each lane handles 8
        // consecutive columns of a row: 16-byte bf16 stores (dgrad), 16-byte
        // stash loads and dG / dU stores (dgrad + dSwiGLU), a quarter of the
        // memory instructions of lane pairs.  Each wavefront stages its 128 x 128
        // float32 sub-tile in two halves of 64 rows in its own 32 KiB of the
        // stage buffers (free once every wave's last loads landed; the barrier
        // at the next tile's claim keeps the next loads out until every wave
        // is done).  A half is [64 rows][32 chunks of 4 floats], chunk c of row
        // r at position c ^ ((c >> 4) & 1) ^ (((r >> 2) & 1) << 3): the
        // MFMA-layout writes (rows r and r + 4 per instruction) and the
        // 8-column reads are both free of bank conflicts.
        // Opaque copies of the tile's first row and of the lane index: the
        // address arithmetic below then stays after the K loop (it is not
        // hoisted out of the tile loop, where it would hold registers).
        int mbase = m0, ln = lane;
        __asm__ volatile("" : "+v"(mbase), "+v"(ln));
        if constexpr (WG) {
            // this wave's last loads (repeats of the last stage) landed before
            // the next tile's loads go out
            __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
            const int N = p.N;
            const int rlim = p.M - mbase;                         // rows of the tile that exist
            const int col = n0 + wn * 128 + (ln & 31);            // + 32 ni
            const int r0 = wm * 128 + 4 * (ln >> 5);              // + 32 mi + 8 (q / 4) + q % 4
            float* const wb = cw + (size_t)mbase * N + col;
            if (rlim >= kTile && n0 + kTile <= N) {  // uniform: a whole tile, no checks
#pragma unroll
                for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                    for (int q = 0; q < 16; ++q) {
                        float* const d = wb + (size_t)(r0 + 32 * mi + 8 * (q >> 2) + (q & 3)) * N;
#pragma unroll
                        for (int ni = 0; ni < 4; ++ni) st_nt(d + 32 * ni, agpr_read(acc[mi][ni][q]));
                    }
            } else {
                bool cok[4];
#pragma unroll
                for (int ni = 0; ni < 4; ++ni) cok[ni] = col + 32 * ni < N;
#pragma unroll
                for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                    for (int q = 0; q < 16; ++q) {
                        const int r = r0 + 32 * mi + 8 * (q >> 2) + (q & 3);
                        float* const d = wb + (size_t)r * N;
                        const bool rok = r < rlim;
#pragma unroll
                        for (int ni = 0; ni < 4; ++ni)
                            if (rok && cok[ni]) st_nt(d + 32 * ni, agpr_read(acc[mi][ni][q]));
                    }
            }
            continue;
        }
        __asm__ volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        const int N = p.N;
        const int rlim = row_end - mbase;  // rows of the tile that exist
        uint8_t* const stg = &lds[0][0][0] + wid * 32768;
        const int hh = ln >> 5, ca = (ln & 31) >> 2;
        uint8_t* wa[4];  // this lane's write address for fragment ni (row 0 of the half)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
            wa[ni] = stg + hh * 2048 + ((((ni ^ hh) << 3) | (ca ^ ((ni >> 1) & 1))) << 4) + (ln & 3) * 4;
        const int kc8 = ln & 15, rq = ln >> 4;  // this lane's column group (8 columns) and row in a pass
        const uint8_t* ra[2][2];                // read addresses [pass parity][lo, hi chunk]
#pragma unroll
        for (int par = 0; par < 2; ++par)
#pragma unroll
            for (int hl = 0; hl < 2; ++hl)
                ra[par][hl] = stg + rq * 512 + ((((2 * kc8 + hl) ^ (kc8 >> 3)) ^ (par << 3)) << 4);
        const int ncol = n0 + wn * 128 + 8 * kc8;  // this lane's first column
        const bool col_ok = ncol < N;
        // row 0 of the tile at this lane's columns: dgrad (bf16, N per row),
        // dgrad + dSwiGLU (bf16, 2N per row, stash alike)
        const int ldc = DSW ? 2 * N : N;
        uint16_t* const cbase = p.C + (size_t)mbase * ldc + ncol;
        const uint16_t* const sbase = DSW ? p.stash + (size_t)mbase * ldc + ncol : nullptr;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            // dgrad + dSwiGLU: stash rows of the half's 16 passes (4 rows each)
            // through a ring of 8: passes 0..7 are loaded before the staging,
            // pass p + 8 right after pass p is consumed
            uint4 gq[8], uq[8];
#define GB_LOAD_STASH(PS)                                                                                \
    {                                                                                                    \
        const int r_ = wm * 128 + hf * 64 + 4 * (PS) + rq;                                               \
        if (col_ok && r_ < rlim) {                                                                       \
            gq[(PS) & 7] = *(const uint4*)(sbase + (size_t)r_ * ldc);                                    \
            uq[(PS) & 7] = *(const uint4*)(sbase + (size_t)r_ * ldc + N);                                \
        }                                                                                                \
    }
            if (DSW) {
#pragma unroll
                for (int ps = 0; ps < 8; ++ps) GB_LOAD_STASH(ps)
            }
#pragma unroll
            for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
                for (int ni = 0; ni < 4; ++ni)
#pragma unroll
                    for (int q = 0; q < 16; ++q)
                        *(float*)(wa[ni] + (32 * m2 + 8 * (q >> 2) + (q & 3)) * 512) =
                            agpr_read(acc[2 * hf + m2][ni][q]);
#pragma unroll
            for (int ps = 0; ps < 16; ++ps) {
                const int r = wm * 128 + hf * 64 + 4 * ps + rq;
                const bool ok = col_ok && r < rlim;
                const float4 lo = *(const float4*)(ra[ps & 1][0] + ps * 2048);
                const float4 hi = *(const float4*)(ra[ps & 1][1] + ps * 2048);
                if (MODE == kDgrad) {
                    if (ok)
                        st_nt((uint4*)(cbase + (size_t)r * ldc), make_uint4(
                            pack_bf16x2(lo.x, lo.y), pack_bf16x2(lo.z, lo.w), pack_bf16x2(hi.x, hi.y),
                            pack_bf16x2(hi.z, hi.w)));
                } else {
                    const float dh[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                    const uint32_t gw[4] = {gq[ps & 7].x, gq[ps & 7].y, gq[ps & 7].z, gq[ps & 7].w};
                    const uint32_t uw[4] = {uq[ps & 7].x, uq[ps & 7].y, uq[ps & 7].z, uq[ps & 7].w};
                    if (ps < 8) GB_LOAD_STASH(ps + 8)
                    uint32_t dg[4], du[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        float rg[2], ru[2];
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            float g = __uint_as_float(h ? (gw[j] & 0xffff0000u) : (gw[j] << 16));
                            float u = __uint_as_float(h ? (uw[j] & 0xffff0000u) : (uw[j] << 16));
                            // a = dh sigma(g); dU = a g; dG = a u (1 + g (1 - sigma(g)))
                            if constexpr (MODE == kDgradDswigluClamp) {
                                const bool kg = !(g > p.lim), ku = !(u > p.lim || u < -p.lim);
                                g = fminf(g, p.lim);
                                u = fminf(fmaxf(u, -p.lim), p.lim);
                                const float sg = sigmoid_fast(g);
                                const float a = dh[2 * j + h] * sg;
                                rg[h] = kg ? a * u * fmaf(g, 1.0f - sg, 1.0f) : 0.f;
                                ru[h] = ku ? a * g : 0.f;
                            } else {
                                const float sg = sigmoid_fast(g);
                                const float a = dh[2 * j + h] * sg;
                                rg[h] = a * u * fmaf(g, 1.0f - sg, 1.0f);
                                ru[h] = a * g;
                            }
                        }
                        dg[j] = pack_bf16x2(rg[0], rg[1]);
                        du[j] = pack_bf16x2(ru[0], ru[1]);
                    }
                    if (ok) {
                        st_nt((uint4*)(cbase + (size_t)r * ldc), make_uint4(dg[0], dg[1], dg[2], dg[3]));
                        st_nt((uint4*)(cbase + (size_t)r * ldc + N), make_uint4(du[0], du[1], du[2], du[3]));
                    }
                }
            }
#undef GB_LOAD_STASH
        }
    }
}

}  // namespace gemm
}  // namespace moe
