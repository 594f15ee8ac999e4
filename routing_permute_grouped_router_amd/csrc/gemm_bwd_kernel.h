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
    constexpr int OPB = kTile * BK * 2;  // bytes of one operand in one stage
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2][2][OPB];
    __shared__ int32_t pre[kMaxExperts + 1];
    __shared__ int32_t spre[WG ? kMaxExperts + 1 : 1];
    __shared__ int scan_tmp[kThreads / 64];

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
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

#define GB_LOAD(kt, st)                                                                                   \
    _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                                       \
        size_t ao = aoff[i] + (size_t)(kt) * a_kstep, bo = boff[i] + (size_t)(kt) * b_kstep;              \
        if (WG) {                                                                                         \
            const int kr = (kt) * BK + 16 * wid + 2 * i + s_kr;                                           \
            if (kr > a_rowcap) {                                                                          \
                const size_t back = (size_t)(kr - a_rowcap);                                              \
                ao -= back * p.M * 2;                                                                     \
                bo -= back * p.N * 2;                                                                     \
            }                                                                                             \
        }                                                                                                 \
        __builtin_amdgcn_global_load_lds((glb_void*)(abase + ao),                                         \
                                         (lds_void*)&lds[st][0][(WG ? (16 * wid + 2 * i) * 512            \
                                                                    : (wid * 64 + 8 * i) * 128)], 16, 0, 0); \
        __builtin_amdgcn_global_load_lds((glb_void*)(bbase + bo),                                         \
                                         (lds_void*)&lds[st][1][(16 * wid + 2 * i) * 512], 16, 0, 0);     \
    }
        // WGRAD tail: zero the A copy of K rows past the unit's end (this wave's own rows, after its loads landed)
#define GB_ZERO_TAIL(kt, st)                                                                              \
    if (WG && (kt) * BK + BK - 1 > a_rowcap) {                                                            \
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");                                             \
        _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                                   \
            const int kr = 16 * wid + 2 * i + s_kr;                                                       \
            if ((kt) * BK + kr > a_rowcap) *(uint4*)&lds[st][0][kr * 512 + s_pos * 16] = make_uint4(0, 0, 0, 0); \
        }                                                                                                 \
    }

        const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void*)&lds[0][0][0];
        // fragments of K sub-step kk (16 values) of the stage in buffer st
#define GB_READ(st, kk, FA, FB)                                                                           \
    {                                                                                                     \
        const uint32_t sa_ = lds_base + (st) * 2 * OPB, sb_ = sa_ + OPB;                                  \
        _Pragma("unroll") for (int mi = 0; mi < 4; ++mi) {                                                \
            if (WG) FA[mi] = bwd_tr_frag(sa_ + a_tr[mi] + (16 * (kk) + 8 * half) * 512);                  \
            else FA[mi] = __builtin_bit_cast(bf16x8, bwd_ds_read16(sa_ + arow[mi] * 128 +                 \
                                                                   ((((kk) * 2 + half) ^ (arow[mi] & 7)) << 4))); \
        }                                                                                                 \
        _Pragma("unroll") for (int ni = 0; ni < 4; ++ni)                                                  \
            FB[ni] = bwd_tr_frag(sb_ + b_tr[ni] + (16 * (kk) + 8 * half) * 512);                          \
    }
#define GB_MFMAS(FA, FB)                                                                                  \
    _Pragma("unroll") for (int mi = 0; mi < 4; ++mi) _Pragma("unroll") for (int ni = 0; ni < 4; ++ni)     \
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(FA[mi], FB[ni], acc[mi][ni], 0, 0, 0);

        bf16x8 f0a[4], f0b[4], f1a[4], f1b[4];
        if (nk > 0) {
            __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");  // previous tile's stores retired
            GB_LOAD(0, 0);
            GB_ZERO_TAIL(0, 0);
            __asm__ volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
            GB_READ(0, 0, f0a, f0b);
            BWD_WAIT(f0a, f0b);
        }
        for (int kt = 0; kt < nk; ++kt) {
            const int st = kt & 1;
            __builtin_amdgcn_sched_barrier(0);
            if (kt + 1 < nk) GB_LOAD(kt + 1, st ^ 1);  // into the buffer freed by the last barrier
            GB_READ(st, 1, f1a, f1b);
            __builtin_amdgcn_sched_barrier(0);
            GB_MFMAS(f0a, f0b);
            __builtin_amdgcn_sched_barrier(0);
            BWD_WAIT(f1a, f1b);
            GB_READ(st, 2, f0a, f0b);
            __builtin_amdgcn_sched_barrier(0);
            GB_MFMAS(f1a, f1b);
            __builtin_amdgcn_sched_barrier(0);
            BWD_WAIT(f0a, f0b);
            GB_READ(st, 3, f1a, f1b);
            __builtin_amdgcn_sched_barrier(0);
            GB_MFMAS(f0a, f0b);
            __builtin_amdgcn_sched_barrier(0);
            BWD_WAIT(f1a, f1b);  // this wave has read all of stage kt
            if (kt + 1 < nk) GB_ZERO_TAIL(kt + 1, st ^ 1);
            // next stage landed for every wave; every wave is done with stage kt
            __asm__ volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            if (kt + 1 < nk) GB_READ(st ^ 1, 0, f0a, f0b);
            __builtin_amdgcn_sched_barrier(0);
            GB_MFMAS(f1a, f1b);
            __builtin_amdgcn_sched_barrier(0);
            if (kt + 1 < nk) BWD_WAIT(f0a, f0b);
        }
#undef GB_READ
#undef GB_MFMAS
#undef GB_LOAD
#undef GB_ZERO_TAIL
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
