// Grouped bf16 GEMM kernel template for CDNA4 (v_mfma_f32_16x16x32_bf16).
//
// C[r, n] = sum_k A[r, k] * B_e[n, k] for the rows r of expert e, group sizes
// read from the device `offsets` buffer.  Both operands have K contiguous (rows
// of Xp or h, and the stored weights), so every global load is 16 bytes and
// every MFMA operand is one 16-byte LDS read.
//
// Block: 256 threads = 4 wavefronts in a 2 x 2 grid; tile 256 x 256 x 64; each
// wavefront owns a 128 x 128 sub-tile held in 8 x 8 MFMA 16x16 accumulators
// (256 accumulator registers per lane).  Operand tiles go from global memory
// straight into LDS with global_load_lds_dwordx4 (lane i of one load lands at
// LDS base + 16 i), two stages of 64 KiB, so stage k+2 streams in while stages
// k and k+1 feed the matrix cores.  In LDS each row's 16-byte K chunks are XOR-
// permuted by a function of the row (swz) so that the MFMA operand reads of
// consecutive rows hit distinct banks; the permutation is applied on the global
// side (a lane fetches the chunk its LDS slot must hold).  Rows past a group's
// end, and columns past the output width, load a clamped valid row and are
// never stored.
//
// SwiGLU tiles put 128 gate rows (f0..f0+127) and the matching 128 up rows
// (F+f0..) of W1 in one 256-row B tile; a wavefront's accumulators (mi, ni) and
// (mi, ni+4) are then gate and up of the same outputs in the same lanes, and
// the epilogue forms silu(g) * u in registers.
//
// The grid is persistent (one block per CU); block b runs on XCD b % 8 and
// the tile sequence (expert by expert; tile_of) is cut into 8 contiguous
// ranges, one per XCD, so the blocks of an XCD share A rows and B columns in
// its L2; the blocks take their units through per-XCD work queues (below).
#pragma once

#include <type_traits>

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
    int* sched;             // [kXcds] work-queue counters, zero at launch
    float* part;            // [kXcds * kSlotsPerXcd][kTile][kTile] partial sums of split tiles
    // Gather (gate/up GEMM only; src_map null otherwise): A is x [T, K] and row
    // r of the grouped operand is x[src_map[r] / gk]; the first counts[e] rows
    // of expert e are routed, the rest of its group are padding rows, whose
    // outputs are stored as zeros (as for the zero rows of a materialised Xp).
    const int32_t* src_map;
    const int32_t* counts;
    int gk;
    // Optional per-row routing weights (the epilogue placements of the
    // weight): output row r is scaled by row_w[r] before it is stored.  The
    // array holds 256 rows past `rows`, so a tile reads without a bound.
    const float* row_w;
    // SwiGLU clamp limit (the clamped variant only): g <- min(g, lim),
    // u <- clamp(u, -lim, lim) before the activation; +inf when off
    float lim;
};

// Work queues.  The tiles are cut into kXcds contiguous ranges, one per XCD
// (block b runs on XCD b % kXcds).  The blocks of an XCD take work units from
// their range in order through an atomic counter, so a block that finishes
// early takes more, and once the range is used up they take units from the
// other XCDs' ranges.  When the tiles of a range do not fill the last round of
// the XCD's blocks, its last r tiles are cut along K into S parts each (parts
// of at least kMinSplitStages stages), so the last round is made of shorter
// units; their float32 partial sums go to `part` and split_reduce_bf16 adds
// them in part order and applies the epilogue.
constexpr int kSlotsPerXcd = 32;
constexpr int kMaxSplit = 8;
constexpr int kMinSplitStages = 32;

struct Queue {
    int tb;     // first tile of the range
    int whole;  // units that are whole tiles (the first `whole` tiles)
    int S;      // parts per split tile (1: no split)
    int units;  // whole + split tiles * S
};

// The queue of XCD x: total tiles, nb blocks per XCD, nk K stages per tile.
__device__ __forceinline__ Queue xcd_queue(int total, int x, int nb, int nk) {
    Queue q;
    q.tb = (int)((int64_t)total * x / kXcds);
    const int n = (int)((int64_t)total * (x + 1) / kXcds) - q.tb;
    const int r = n % nb;
    int best = 1;
    if (r > 0) {
        // The last round's work, in tiles, if its r tiles are cut in S parts
        // and the XCD's blocks take them in step: ceil(r S / nb) / S.  Compared
        // exactly (integers), so the reduction kernel makes the same choice.
        int best_rounds = 1;  // ceil(r / nb) for S = 1
        const int smax = min(min(kMaxSplit, nk / kMinSplitStages), kSlotsPerXcd / r);
        for (int S = 2; S <= smax; ++S) {
            const int rounds = (r * S + nb - 1) / nb;
            if (rounds * best < best_rounds * S) {
                best_rounds = rounds;
                best = S;
            }
        }
    }
    q.S = best;
    q.whole = best > 1 ? n - r : n;
    q.units = q.whole + (best > 1 ? r * best : 0);
    return q;
}

// XOR mask applied to a row's 16-byte K chunk index in LDS (CH chunks per
// row).  128-byte rows: mode 0 spreads any 8 consecutive rows over distinct
// banks of a 32-bank LDS, mode 1 also any 16 over a 64-bank one.  64-byte rows
// (two per 128 bytes): the same two guarantees with the row pair folded in.
// Which one suits a kernel depends on how its fragment reads map lanes to
// rows, and was measured (the LDS bank-conflict counter): the bf16 kernel's
// 16x16x32 reads (lane l: row l % 16) are conflict-free with mode 0, while
// mode 2 stalls on conflicts in half of its LDS-active cycles; the MXFP8
// kernel's 32x32x64 reads (lane l: row l % 32) conflict least with mode 1.
template <int SWZ, int CH = 8>
__device__ __forceinline__ int swz(int row) {
    if (CH == 8) {
        if (SWZ == 2) return (row & 7) ^ ((row >> 3) & 1);
        return SWZ == 1 ? ((row ^ (row >> 3)) & 7) : (row & 7);
    }
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

// A 32 x 32 fp32 accumulator tile holds, in lane l and slot q, row
// 8 (q / 4) + 4 (l / 32) + q % 4 of column l % 32.  agpr_read reads one
// element out of its AGPR where it is used, so the compiler does not copy
// every accumulator to VGPRs as the K loop ends.
__device__ __forceinline__ float agpr_read(float a) {
    float v;
    __asm__ volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
    return v;
}

// Output column of B row r of a forward tile (tile-relative).  A wavefront
// reads B fragment ni of its column half wn from LDS rows wn 128 + 32 ni + c
// (c = 0..31), and MFMA lane l holds column c = l % 32 of every fragment; with
// row wn 128 + 32 ni + c carrying output column wn 128 + 4 c + ni, lane l ends
// up with the four adjacent columns 4 c .. 4 c + 3 of each of its rows, one
// from each fragment, and stores them as one 8-byte word with no lane
// exchange.  SwiGLU tiles (gate rows 0..127, up rows 128..255; fragments 0, 1
// of half wn at rows wn 64 + 32 ni + c): h column wn 64 + 2 c + ni, so each
// lane holds two adjacent h columns.
__device__ __forceinline__ int out_col(int r) { return (r & 128) + 4 * (r & 31) + ((r >> 5) & 3); }
__device__ __forceinline__ int out_col_swiglu(int h) { return (h & 64) + 2 * (h & 31) + ((h >> 5) & 1); }

// One 16-byte MFMA operand fragment from LDS.  Issued as inline assembly so
// the compiler neither reorders it nor makes it wait for the direct-to-LDS
// loads into the other stage buffer (it cannot prove that they do not
// alias); the kernel waits for its reads itself (lgkmcnt) before the
// fragments are used.
// Direct global-to-LDS copies.  Lane l copies 16 (or 4) bytes from
// sbase + voff to LDS address lds + 16 l (4 l).  The LDS address is uniform and
// goes through M0 with one scalar move; the global address is a uniform 64-bit
// base plus a 32-bit lane offset.  Any vector arithmetic on the address path
// (64-bit adds, readfirstlane into M0) would sit between the MFMAs of the
// K loop and stall their issue; this form needs none.  Issued as inline
// assembly: the kernel counts these loads itself (vmcnt).
__device__ __forceinline__ void dma_lds16(uint32_t lds, uint32_t voff, const void* sbase) {
    __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(sbase)
                     : "memory", "m0");
}
__device__ __forceinline__ void dma_lds4(uint32_t lds, uint32_t voff, const void* sbase) {
    __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2" ::"s"(lds), "v"(voff), "s"(sbase)
                     : "memory", "m0");
}

// Grouped form of dma_lds16: set_m0 writes M0 once for four loads, and each
// load's immediate offset is added to both its LDS and its global address (a
// one-wavefront check with a padded buffer showed both moving by the offset).
// The grouped GEMM loads four consecutive 1 KiB LDS rows per M0 (offsets 0,
// 1, 2, 3 KiB); its per-lane global offsets carry a bias of 3 KiB minus the
// load's offset and the uniform bases are 3 KiB lower, so every global
// address is the one a plain load would use.  Nothing else in the K loop
// writes M0.
__device__ __forceinline__ void set_m0(uint32_t lds) {
    __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0" ::"s"(lds) : "m0");
}
template <int OFF>
__device__ __forceinline__ void dma_lds16_o(uint32_t voff, const void* sbase) {
    __asm__ volatile("global_load_lds_dwordx4 %0, %1 offset:%2" ::"v"(voff), "s"(sbase), "i"(OFF) : "memory");
}

template <int OFF>
__device__ __forceinline__ bf16x8 lds_frag(uint32_t addr) {
    uint4 v;
    __asm__ volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF) : "memory");
    return __builtin_bit_cast(bf16x8, v);
}

// Nontemporal store of a 1-, 4-, 8- or 16-byte value: GEMM outputs are not
// read again by the kernel that writes them, and leaving them out of the
// cache's working set keeps the operand panels that neighbouring blocks share
// resident in L2.
template <class T>
__device__ __forceinline__ void st_nt(T* p, const T& v) {
    if constexpr (sizeof(T) == 16) {
        typedef unsigned u4v __attribute__((ext_vector_type(4)));
        __builtin_nontemporal_store(__builtin_bit_cast(u4v, v), (u4v*)p);
    } else if constexpr (sizeof(T) == 8) {
        typedef unsigned u2v __attribute__((ext_vector_type(2)));
        __builtin_nontemporal_store(__builtin_bit_cast(u2v, v), (u2v*)p);
    } else {
        __builtin_nontemporal_store(v, p);
    }
}

#ifndef GK_BARRIER_AT
#define GK_BARRIER_AT 40
#endif

// 16x16x32 fragments and accumulators.
typedef float f32x4 __attribute__((ext_vector_type(4)));

// f(std::integral_constant<int, i>) for i = 0 .. N-1, in order (a loop whose
// index is a constant expression in its body).
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, I + 1>(f);
    }
}

// Output column of B row r of a forward tile for the 16x16x32 layout.  A
// wavefront reads B fragment ni of its column half wn from LDS rows
// wn 128 + 16 ni + c (c = 0..15), and MFMA lane l holds column c = l % 16 of
// every fragment; with that row carrying output column wn 128 + 8 c + ni,
// lane l holds the eight adjacent columns 8 c .. 8 c + 7 of each of its rows,
// one per fragment, and stores them as one 16-byte word.  SwiGLU tiles (gate
// rows 0..127, up rows 128..255; gate fragments 0..3 of half wn at rows
// wn 64 + 16 ni + c, up fragments 4..7 the same rows + 128): h column
// wn 64 + 4 c + ni, four adjacent h columns per lane.
__device__ __forceinline__ int out_col16(int r) { return (r & 128) + 8 * (r & 15) + ((r >> 4) & 7); }
__device__ __forceinline__ int out_col16_swiglu(int h) { return (h & 64) + 4 * (h & 15) + ((h >> 4) & 3); }

// EP, epilogue variant bits (built separately, so the plain kernel carries
// none of it): 1 = the outputs are scaled by p.row_w, 2 = the SwiGLU inputs
// are clamped to p.lim.
//
// Block tile 256 x 256 x 64, 4 wavefronts of 128 x 128 in a 2 x 2 grid; a
// wavefront's sub-tile is 8 x 8 v_mfma_f32_16x16x32_bf16 accumulators (256
// accumulator registers).  On MI355X this instruction sustains ~16 % more
// throughput than the 32x32x16 form on Gaussian operands (the part runs at
// its power limit), for the same LDS bytes per flop.  A 64-deep stage is two
// 32-deep K sub-steps of 64 MFMAs.  Chunk c of tile row r is stored at
// position c ^ swz(r); fragments start at multiples of 16 rows, so with
// SWZ 0 or 2 the permutation depends only on the lane.
template <bool SWIGLU, int SWZ, int GM, int EP>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_bf16(Args p) {
    static_assert(SWZ == 0 || SWZ == 2, "the fragment addressing needs a swizzle of the row within 16");
    constexpr int BK = 64;                  // K depth of one stage
    constexpr int CH = BK / 8;              // 16-byte chunks per LDS row
    constexpr int RPL = 64 / CH;            // rows per wave-wide load
    constexpr int LOADS = 64 / RPL;         // loads per wave per operand per stage
    constexpr int STAGE_ELEMS = kTile * BK; // one operand of one stage
    constexpr uint32_t kRowBytes = BK * 2;
    constexpr uint32_t kFragBytes = 16 * kRowBytes;  // one 16-row fragment
    // The stage's first barrier sits before MFMA kBar of its first sub-step;
    // the 16 loads of stage k+2 follow it, one per four MFMAs (kLoads0 of them
    // in the first sub-step, the rest at the start of the second).
    constexpr int kBar = GK_BARRIER_AT;
    constexpr int kLoads0 = (64 - kBar + 3) / 4;
    // A second barrier, before MFMA kBarB of the second sub-step: stage kt+1
    // has landed for every wave, and its first fragments are read after it.
    constexpr int kBarB = 16;

    __shared__ __attribute__((aligned(1024))) uint16_t lds[2][2][STAGE_ELEMS];
    __shared__ int32_t pre[kMaxExperts + 1];
    __shared__ int32_t offs[kMaxExperts + 1];  // the group offsets, read once per block
    __shared__ int scan_tmp[kThreads / 64];
    __shared__ Queue queues[kXcds];
    __shared__ int s_unit;                     // the block's next work unit (thread 0 claims it)

    const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wid >> 1, wn = wid & 1;
    for (int e = tid; e <= p.E; e += kThreads) offs[e] = p.offsets[e];
    const int total_m = build_tile_prefix(p.offsets, p.E, kTile, pre, scan_tmp);  // ends with a barrier
    const int cols_per_tile = SWIGLU ? kTile / 2 : kTile;
    const int n_tiles = (p.n_out + cols_per_tile - 1) / cols_per_tile;  // last N tile may be partial
    const int total = total_m * n_tiles;

    const int K = p.K;
    const int nk = K / BK;
    const int xcd = blockIdx.x % kXcds, nb = gridDim.x / kXcds;
    if (tid < kXcds) queues[tid] = xcd_queue(total, tid, nb, nk);
    // Thread 0 claims units: tickets from the own XCD's queue, then units of
    // the other XCDs' queues once it is used up (a unit is (queue << 20) |
    // index; -1 when every queue is used up).  `dry` remembers the queues
    // found empty, so each costs one atomic.  A ticket is taken one unit ahead
    // and looked at only after the next full memory wait, so no wave waits on
    // the atomic; stealing (only at the end) waits.
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
    // LDS byte addresses of this lane's A and B fragment 0 (stage 0) and the
    // offsets of its chunk in the two K sub-steps: lane l reads row l % 16 of
    // a fragment at chunk 4 kk + l / 16, stored at (4 kk + l / 16) ^ swz(row).
    const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void*)&lds[0][0][0];
    constexpr uint32_t kStageBytes = 2 * STAGE_ELEMS * 2;
    // LDS rows this wave's loads fill: wid * 64 .. +63 of each operand
    const uint32_t lds_wave = __builtin_amdgcn_readfirstlane(lds_base + (uint32_t)(wid * 64) * kRowBytes);
    const int fr = lane & 15;
    const uint32_t a_rd = lds_base + (uint32_t)(wm * 128 + fr) * kRowBytes;
    const uint32_t b_rd = lds_base + (uint32_t)(STAGE_ELEMS * 2) + (uint32_t)((SWIGLU ? wn * 64 : wn * 128) + fr) * kRowBytes;
    const uint32_t koff0 = (uint32_t)((((lane >> 4)) ^ swz<SWZ>(fr)) << 4);
    const uint32_t koff1 = (uint32_t)(((4 + (lane >> 4)) ^ swz<SWZ>(fr)) << 4);
    // State of the unit in flight, set by `setup`: its tile, K stages
    // [kb, ke), partial-sum slot (-1: whole tile), load offsets and bases.
    int kb = 0, ke = 0, slot = -1, row0 = 0, row_end = 0, a_end = 0, nt = 0;
    bool valid = false;
    uint32_t aoff[LOADS], boff[LOADS];
    const char* abase = (const char*)p.A;
    const char* bbase = (const char*)p.B;
    constexpr uint32_t kBias = 3 * RPL * kRowBytes;  // global offsets are biased by this, the bases lowered
#define GK_LOAD_A(kt, stage, i)                                                                          \
    {                                                                                                    \
        if constexpr ((i) % 4 == 0) set_m0(lds_wave + (uint32_t)(stage) * kStageBytes + (i) * RPL * kRowBytes); \
        dma_lds16_o<((i) % 4) * RPL * kRowBytes>(aoff[i], abase + (size_t)(kt) * (BK * 2));              \
    }
#define GK_LOAD_B(kt, stage, i)                                                                          \
    {                                                                                                    \
        if constexpr ((i) % 4 == 0)                                                                      \
            set_m0(lds_wave + (uint32_t)(stage) * kStageBytes + STAGE_ELEMS * 2 + (i) * RPL * kRowBytes);  \
        dma_lds16_o<((i) % 4) * RPL * kRowBytes>(boff[i], bbase + (size_t)(kt) * (BK * 2));              \
    }
// B fragment ni's byte offset from fragment 0 (SwiGLU: up fragments 4..7 are
// the gate fragments' rows + 128)
#define GK_BOFF(ni) (SWIGLU ? ((ni) & 3) * kFragBytes + ((ni) >> 2) * 128 * kRowBytes : (ni) * kFragBytes)
#define GK_SB __builtin_amdgcn_sched_barrier(0)

    // Decode unit u (from `take`), compute its tile's addressing and issue
    // the loads of its first two stages (stage buffers 0 and 1).  Called right
    // after the previous unit's K loop, so these loads are in flight while
    // that unit's epilogue runs.
    auto setup = [&](int u) __attribute__((always_inline)) {
        u = __builtin_amdgcn_readfirstlane(u);
        if (u < 0) {  // no unit (every queue used up): nothing to decode or load
            valid = false;
            kb = ke = 0;
            return;
        }
        const int ux = __builtin_amdgcn_readfirstlane(u >> 20), uu = __builtin_amdgcn_readfirstlane(u & 0xFFFFF);
        const Queue q = queues[ux];
        int t;
        kb = 0;
        ke = nk;
        slot = -1;
        if (uu < q.whole) {
            t = q.tb + uu;
        } else {
            const int j = uu - q.whole;
            t = q.tb + q.whole + j / q.S;
            const int part = j % q.S;
            kb = part * nk / q.S;
            ke = (part + 1) * nk / q.S;
            slot = ux * kSlotsPerXcd + j;
        }
        t = __builtin_amdgcn_readfirstlane(t);
        kb = __builtin_amdgcn_readfirstlane(kb);
        ke = __builtin_amdgcn_readfirstlane(ke);
        slot = __builtin_amdgcn_readfirstlane(slot);
        int mt, ntt, ee;
        tile_of(t, pre, p.E, total_m, n_tiles, GM, &ee, &mt, &ntt);
        nt = __builtin_amdgcn_readfirstlane(ntt);
        mt = __builtin_amdgcn_readfirstlane(mt);
        const int e = __builtin_amdgcn_readfirstlane(ee);
        row_end = __builtin_amdgcn_readfirstlane(min(offs[e + 1], p.rows));
        row0 = __builtin_amdgcn_readfirstlane(offs[e] + (mt - pre[e]) * kTile);
        // row0 outside [0, row_end) only happens for inconsistent offsets: the
        // unit is then skipped (no loads, no K loop, nothing stored)
        valid = row0 >= 0 && row0 < row_end;
        if (!valid) {
            kb = ke = 0;
            return;
        }
        // rows with an A row of their own: all, or (gather) the routed rows
        a_end = p.src_map ? __builtin_amdgcn_readfirstlane(min(offs[e] + p.counts[e], row_end)) : row_end;
        // first B row of the tile (SwiGLU: first gate row; the up rows are F rows further)
        const int brow0 = SWIGLU ? nt * 128 : nt * kTile;
        // Per-lane byte offsets of the A and B loads (K offset 0) against the
        // uniform tile bases: 32-bit, so the loads take few registers.  They
        // are formed from an opaque copy of the lane index, so the compiler
        // recomputes them per tile instead of holding per-lane constants
        // across the K loop.
        int sl = lane;
        __asm__ volatile("" : "+v"(sl));
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int r = wid * 64 + i * RPL + sl / CH;  // tile row 0..255
            const int chunk = (sl % CH) ^ swz<SWZ>(r);
            const int ar = min(row0 + r, a_end - 1);
            aoff[i] = p.src_map ? (uint32_t)(((size_t)(p.src_map[ar] / p.gk) * K + chunk * 8) * 2)
                                : (uint32_t)(((size_t)(ar - row0) * K + chunk * 8) * 2);
            int br;
            if (SWIGLU) {
                const int f = min(nt * 128 + out_col16_swiglu(r & 127), p.n_out - 1);
                br = r < 128 ? f : p.n_out + f;
            } else {
                br = min(nt * kTile + out_col16(r), p.n_out - 1);
            }
            boff[i] = (uint32_t)(((size_t)(br - brow0) * K + chunk * 8) * 2);
            aoff[i] += kBias - (uint32_t)((i % 4) * RPL * kRowBytes);
            boff[i] += kBias - (uint32_t)((i % 4) * RPL * kRowBytes);
        }
        abase = (p.src_map ? (const char*)p.A : (const char*)(p.A + (size_t)row0 * K)) - kBias;
        bbase = (const char*)(p.B + ((size_t)e * p.b_rows + brow0) * K) - kBias;
        GK_SB;
        static_for<LOADS>([&](auto ic) __attribute__((always_inline)) { GK_LOAD_B(kb, 0, decltype(ic)::value); });
        static_for<LOADS>([&](auto ic) __attribute__((always_inline)) { GK_LOAD_A(kb, 0, decltype(ic)::value); });
        if (kb + 1 < ke) {
            static_for<LOADS>([&](auto ic) __attribute__((always_inline)) { GK_LOAD_B(kb + 1, 1, decltype(ic)::value); });
            static_for<LOADS>([&](auto ic) __attribute__((always_inline)) { GK_LOAD_A(kb + 1, 1, decltype(ic)::value); });
        }
        GK_SB;
    };

    setup(unit);
    while (unit >= 0) {
        // Two LDS stage buffers.  Iteration kt (buffer st holds stage kt, the
        // other buffer stage kt+1, landed or in flight):
        //   sub-step 0: 64 MFMAs on the fragments fx (K 0..31 of stage kt),
        //     the 16 fragment reads of K 32..63 into fy under the first 32;
        //     then each wave has read all of stage kt (lgkmcnt), and past the
        //     barrier that holds for every wave: buffer st is free.  The 16
        //     loads of stage kt+2 into buffer st start there, B (the weights,
        //     first touched in HBM) before A, one per four MFMAs;
        //   sub-step 1: 64 MFMAs on fy and the rest of those loads; before
        //     MFMA kBarB each wave waits for its loads of stage kt+1 (those of
        //     stage kt+2 may stay in flight), and past a second barrier stage
        //     kt+1 is readable for every wave: the 16 fragment reads of its K
        //     0..31 into fx follow.  Waiting for stage kt+1 there rather than at
        //     the first barrier gives its last loads ~100 MFMAs instead of ~70
        //     to land.
        // One load per four MFMAs per wave is about what the CU's address unit
        // sustains for the four wavefronts.  There are no loads past K.
        bf16x8 fxa[8], fxb[8], fya[8], fyb[8];
        // the unit's first stage landed everywhere; the previous unit's stores retired
        __asm__ volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        GK_SB;
        if (tid == 0) {  // publish the next unit, take a ticket for the one after
            const int nu = take(tick);
            s_unit = nu;
            tick = nu >= 0 ? ticket() : -1;
        }
        // The accumulators live in the accumulator registers for the whole tile:
        // empty asm statements with "a" constraints (at the zeroing and once
        // per K iteration) keep the register allocator from moving some of
        // them to VGPRs and copying them around the MFMAs.
        f32x4 acc[8][8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) __asm__ volatile("" : "=a"(acc[i][j]) : "0"((f32x4){0.f, 0.f, 0.f, 0.f}));
#define GK_PIN_ACC(I)                                                                                    \
    __asm__ volatile("" : "+a"(acc[I][0]), "+a"(acc[I][1]), "+a"(acc[I][2]), "+a"(acc[I][3]),            \
                     "+a"(acc[I][4]), "+a"(acc[I][5]), "+a"(acc[I][6]), "+a"(acc[I][7]))
        static_for<8>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            fxa[i] = lds_frag<i * kFragBytes>(a_rd + koff0);
            fxb[i] = lds_frag<GK_BOFF(i)>(b_rd + koff0);
        });
#define GK_WAIT_FRAGS(FA, FB)                                                                            \
    __asm__ volatile("s_waitcnt lgkmcnt(0)"                                                              \
                     : "+v"(FA[0]), "+v"(FA[1]), "+v"(FA[2]), "+v"(FA[3]), "+v"(FA[4]), "+v"(FA[5]),     \
                       "+v"(FA[6]), "+v"(FA[7]), "+v"(FB[0]), "+v"(FB[1]), "+v"(FB[2]), "+v"(FB[3]),     \
                       "+v"(FB[4]), "+v"(FB[5]), "+v"(FB[6]), "+v"(FB[7])::"memory")
        GK_WAIT_FRAGS(fxa, fxb);
        // One iteration of the K loop; LD: whether it loads stage kt+2 (the
        // loop is split so that no branch sits between the MFMAs).
        auto iteration = [&](int kt, auto ld) __attribute__((always_inline)) {
            constexpr bool LD = decltype(ld)::value;
            const int st = (kt - kb) & 1;
            const uint32_t so = (uint32_t)st * kStageBytes, nso = so ^ kStageBytes;
            const int lkt = kt + 2;
            GK_PIN_ACC(0); GK_PIN_ACC(1); GK_PIN_ACC(2); GK_PIN_ACC(3);
            GK_PIN_ACC(4); GK_PIN_ACC(5); GK_PIN_ACC(6); GK_PIN_ACC(7);
            // fragment j (0..15: A 0..7, B 0..7) of the K half at KOFF of the stage at byte offset SO
#define GK_READ(FA, FB, SO, KOFF, j)                                                                     \
    if constexpr ((j) < 8) FA[(j)] = lds_frag<(j) * kFragBytes>(a_rd + (SO) + (KOFF));                   \
    else FB[(j) - 8] = lds_frag<GK_BOFF((j) - 8)>(b_rd + (SO) + (KOFF));
            // load j (0..15: B 0..7, then A 0..7) of stage kt+2 into buffer st
#define GK_LOAD(j)                                                                                       \
    if constexpr (LD) {                                                                                  \
        if constexpr ((j) < 8) { GK_LOAD_B(lkt, st, (j)); }                                              \
        else { GK_LOAD_A(lkt, st, (j) - 8); }                                                            \
    }
            GK_SB;
            // sub-step 0
            static_for<64>([&](auto mc) __attribute__((always_inline)) {
                constexpr int m = decltype(mc)::value;
                if constexpr (m == kBar) {
                    // own reads of stage kt done; then for every wave (buffer st is free)
                    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier"
                                     : "+v"(fya[0]), "+v"(fya[1]), "+v"(fya[2]), "+v"(fya[3]), "+v"(fya[4]),
                                       "+v"(fya[5]), "+v"(fya[6]), "+v"(fya[7]), "+v"(fyb[0]), "+v"(fyb[1]),
                                       "+v"(fyb[2]), "+v"(fyb[3]), "+v"(fyb[4]), "+v"(fyb[5]), "+v"(fyb[6]),
                                       "+v"(fyb[7])::"memory");
                    GK_SB;
                }
                if constexpr (m >= kBar && ((m - kBar) & 3) == 0) {
                    GK_LOAD((m - kBar) / 4)
                }
                acc[m >> 3][m & 7] =
                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(fxa[m >> 3], fxb[m & 7], acc[m >> 3][m & 7], 0, 0, 0);
                if constexpr (m < 32 && (m & 1) == 0) {
                    GK_READ(fya, fyb, so, koff1, m / 2)
                }
                GK_SB;
            });
            // sub-step 1 (after the last stage the reads of "stage kt+1" fetch
            // unused bytes of the other buffer)
            static_for<64>([&](auto mc) __attribute__((always_inline)) {
                constexpr int m = decltype(mc)::value;
                if constexpr (m == kBarB) {
                    // own loads of stage kt+1 landed: the loads of stage kt+2
                    // issued so far are younger, and vector memory operations
                    // complete in issue order; then for every wave
                    if constexpr (LD) {
                        static_assert(kLoads0 + (kBarB + 3) / 4 == 10, "the count below is the loads issued so far");
                        __asm__ volatile("s_waitcnt vmcnt(10)\n\ts_barrier" ::: "memory");
                    } else {
                        __asm__ volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
                    }
                    GK_SB;
                }
                if constexpr ((m & 3) == 0 && m / 4 < 16 - kLoads0) {
                    GK_LOAD(kLoads0 + m / 4)
                }
                acc[m >> 3][m & 7] =
                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(fya[m >> 3], fyb[m & 7], acc[m >> 3][m & 7], 0, 0, 0);
                if constexpr (m > kBarB && m < kBarB + 32 && ((m - kBarB) & 1) == 1) {
                    GK_READ(fxa, fxb, nso, koff0, (m - kBarB) / 2)
                }
                GK_SB;
            });
            // the next stage's first fragments landed (waiting here rather than at
            // the top of the next iteration leaves no LDS read in flight when the
            // loop ends)
            GK_WAIT_FRAGS(fxa, fxb);
#undef GK_READ
#undef GK_LOAD
        };
        int kt = kb;
        for (; kt + 2 < ke; ++kt) iteration(kt, std::true_type{});
        for (; kt < ke; ++kt) iteration(kt, std::false_type{});
        GK_SB;
#undef GK_LOAD_A
#undef GK_LOAD_B
#undef GK_BOFF
#undef GK_SB
#undef GK_WAIT_FRAGS
#undef GK_PIN_ACC

        // The next unit (published by thread 0 before this unit's K loop; the
        // barrier makes it visible even when the loop had no stage), its
        // first loads issued before this unit's epilogue.
        __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        const int next_unit = s_unit;
        const int e_row0 = row0, e_row_end = row_end, e_a_end = a_end, e_nt = nt, e_slot = slot;
        const bool e_valid = valid;
        // Routing weights of this wave's 128 rows, two per lane (rows 2 lane
        // and 2 lane + 1 of the band), loaded and waited for before setup
        // issues the next unit's loads: the wait then covers only these.
        float rwa = 1.f, rwb = 1.f;
        if constexpr ((EP & 1) != 0) {
            if (e_valid) {
                const float* const rwp = p.row_w + e_row0 + wm * 128 + 2 * lane;
                rwa = rwp[0];
                rwb = rwp[1];
            }
            __asm__ volatile("" : "+v"(rwa), "+v"(rwb));
        }
        if (next_unit >= 0) setup(next_unit);
        if (e_valid) {
        // Epilogue straight from the accumulators.  Lane l holds, in block mi
        // (16 rows) and slot q, row 16 mi + 4 (l / 16) + q of column l % 16 of
        // each fragment; with the B row order above those are 8 adjacent
        // output columns (SwiGLU: 4 h columns).  Opaque copies of the tile's
        // first row and of the lane index keep the address arithmetic after
        // the K loop.
        int rbase = e_row0, ln = lane;
        __asm__ volatile("" : "+v"(rbase), "+v"(ln));
        const int lc = ln & 15;             // this lane's column group
        const int lr = 4 * (ln >> 4);       // this lane's first row in a 16-row block
        const int rlim = e_row_end - rbase;  // rows of the tile that exist
        const int alim = e_a_end - rbase;    // rows of the tile that are not padding (gather)
        // RW[q]: the routing weight of the lane's row q of block MI (1
        // without weights); row i of the wave's band sits in lane i / 2, as
        // rwa (even i) or rwb (odd i).
#define GB_ROW_WEIGHTS(MI, W_)                                                                           \
    if constexpr ((EP & 1) != 0) {                                                                       \
        _Pragma("unroll") for (int q = 0; q < 4; ++q)                                                    \
            W_[q] = __shfl((q & 1) ? rwb : rwa, ((MI) * 16 + lr + q) >> 1, 64);                          \
    } else {                                                                                             \
        _Pragma("unroll") for (int q = 0; q < 4; ++q) W_[q] = 1.f;                                       \
    }
// Store W[q] (type T) to row q past DST (LD elements per row) for q = 0..3:
// the lane's rows of the 16-row block at tile row RB0; rows are checked only
// when the block runs past the group's end.  Nontemporal (st_nt).
#define GB_STORE_ROWS(T, DST, LD, RB0, W)                                                                \
    if ((RB0) + 16 <= rlim) {                                                                            \
        _Pragma("unroll") for (int q = 0; q < 4; ++q) st_nt((T*)((DST) + (size_t)q * (LD)), (W)[q]);      \
    } else {                                                                                             \
        _Pragma("unroll") for (int q = 0; q < 4; ++q)                                                    \
            if ((RB0) + lr + q < rlim) st_nt((T*)((DST) + (size_t)q * (LD)), (W)[q]);                     \
    }

        if (e_slot >= 0) {
            // a K part of a split tile: its float32 partial sums, all 256 x 256
            // (rows past the group's end and columns past the output width
            // included; the reduction skips them), in [row][column] order with
            // SwiGLU gate columns 0..127 and up columns 128..255
            float* const pb = p.part + (size_t)e_slot * kTile * kTile;
            static_for<8>([&](auto ic) __attribute__((always_inline)) {
                constexpr int mi = decltype(ic)::value;
                const int rb0 = wm * 128 + mi * 16;
                float* const prow = pb + (size_t)(rb0 + lr) * kTile;
                if constexpr (SWIGLU) {
                    float4 gw[4], uw[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        gw[q] = make_float4(agpr_read(acc[mi][0][q]), agpr_read(acc[mi][1][q]),
                                            agpr_read(acc[mi][2][q]), agpr_read(acc[mi][3][q]));
                        uw[q] = make_float4(agpr_read(acc[mi][4][q]), agpr_read(acc[mi][5][q]),
                                            agpr_read(acc[mi][6][q]), agpr_read(acc[mi][7][q]));
                    }
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float* const d = prow + (size_t)q * kTile + wn * 64 + 4 * lc;
                        *(float4*)d = gw[q];
                        *(float4*)(d + 128) = uw[q];
                    }
                } else {
                    float4 w0[4], w1[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        w0[q] = make_float4(agpr_read(acc[mi][0][q]), agpr_read(acc[mi][1][q]),
                                            agpr_read(acc[mi][2][q]), agpr_read(acc[mi][3][q]));
                        w1[q] = make_float4(agpr_read(acc[mi][4][q]), agpr_read(acc[mi][5][q]),
                                            agpr_read(acc[mi][6][q]), agpr_read(acc[mi][7][q]));
                    }
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float* const d = prow + (size_t)q * kTile + wn * 128 + 8 * lc;
                        *(float4*)d = w0[q];
                        *(float4*)(d + 4) = w1[q];
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            });
        } else if constexpr (SWIGLU) {
            uint16_t* const cbase = p.C + (size_t)rbase * p.n_out;
            uint16_t* const sbase = p.stash ? p.stash + (size_t)rbase * 2 * p.n_out : nullptr;
            const int f = e_nt * 128 + wn * 64 + 4 * lc;  // this lane's h columns f .. f + 3
            static_for<8>([&](auto ic) __attribute__((always_inline)) {
                constexpr int mi = decltype(ic)::value;
                const int rb0 = wm * 128 + mi * 16;
                uint2 hw[4];
                float rw[4];
                GB_ROW_WEIGHTS(mi, rw)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float g[4], u[4], hv[4];
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        g[c] = agpr_read(acc[mi][c][q]);
                        u[c] = agpr_read(acc[mi][4 + c][q]);
                        if constexpr ((EP & 2) != 0) {
                            g[c] = fminf(g[c], p.lim);
                            u[c] = fminf(fmaxf(u[c], -p.lim), p.lim);
                        }
                        hv[c] = silu(g[c]) * u[c] * rw[q];
                    }
                    hw[q] = make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
                    if (rb0 + lr + q >= alim) hw[q] = make_uint2(0u, 0u);  // gather: padding rows
                }
                if (f < p.n_out) {
                    uint16_t* const dst = cbase + (size_t)(rb0 + lr) * p.n_out + f;
                    GB_STORE_ROWS(uint2, dst, p.n_out, rb0, hw)
                    if (sbase) {
                        uint2 gw[4], uw[4];
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            gw[q] = make_uint2(pack_bf16x2(agpr_read(acc[mi][0][q]), agpr_read(acc[mi][1][q])),
                                               pack_bf16x2(agpr_read(acc[mi][2][q]), agpr_read(acc[mi][3][q])));
                            uw[q] = make_uint2(pack_bf16x2(agpr_read(acc[mi][4][q]), agpr_read(acc[mi][5][q])),
                                               pack_bf16x2(agpr_read(acc[mi][6][q]), agpr_read(acc[mi][7][q])));
                        }
                        uint16_t* const gd = sbase + (size_t)(rb0 + lr) * 2 * p.n_out + f;
                        GB_STORE_ROWS(uint2, gd, 2 * p.n_out, rb0, gw)
                        uint16_t* const ud = gd + p.n_out;
                        GB_STORE_ROWS(uint2, ud, 2 * p.n_out, rb0, uw)
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            });
        } else {
            uint16_t* const cbase = p.C + (size_t)rbase * p.n_out;
            const int n = e_nt * kTile + wn * 128 + 8 * lc;  // this lane's columns n .. n + 7
            static_for<8>([&](auto ic) __attribute__((always_inline)) {
                constexpr int mi = decltype(ic)::value;
                const int rb0 = wm * 128 + mi * 16;
                uint4 w[4];
                float rw[4];
                GB_ROW_WEIGHTS(mi, rw)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float v[8];
#pragma unroll
                    for (int c = 0; c < 8; ++c) v[c] = agpr_read(acc[mi][c][q]) * rw[q];
                    w[q] = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                                      pack_bf16x2(v[6], v[7]));
                }
                if (n < p.n_out) {
                    uint16_t* const dst = cbase + (size_t)(rb0 + lr) * p.n_out + n;
                    GB_STORE_ROWS(uint4, dst, p.n_out, rb0, w)
                }
                __builtin_amdgcn_sched_barrier(0);
            });
        }
#undef GB_STORE_ROWS
#undef GB_ROW_WEIGHTS
        }  // valid
        unit = next_unit;
    }
}

}  // namespace gemm
}  // namespace moe
