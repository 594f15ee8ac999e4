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
// the tile sequence (expert by expert; tile_of) is cut into 8 contiguous
// ranges, one per XCD, so the blocks of an XCD share A rows and B columns in
// its L2; the blocks take their units through per-XCD work queues (below).
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

template <int OFF>
__device__ __forceinline__ bf16x8 lds_frag(uint32_t addr) {
    uint4 v;
    __asm__ volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF) : "memory");
    return __builtin_bit_cast(bf16x8, v);
}

// EP, epilogue variant bits (built separately, so the plain kernel carries
// none of it): 1 = the outputs are scaled by p.row_w, 2 = the SwiGLU inputs
// are clamped to p.lim.
template <bool SWIGLU, int SWZ, int GM, int EP>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_bf16(Args p) {
    constexpr int BK = 64;                  // K depth of one stage
    constexpr int CH = BK / 8;              // 16-byte chunks per LDS row
    constexpr int RPL = 64 / CH;            // rows per wave-wide load
    constexpr int LOADS = 64 / RPL;         // loads per wave per operand per stage
    constexpr int STAGE_ELEMS = kTile * BK; // one operand of one stage
    // byte offsets of B fragments 1..3 from fragment 0: SwiGLU tiles hold
    // gate rows 0..127 and up rows 128..255 (fragments 2, 3 are the up rows
    // of fragments 0, 1); other tiles 32 consecutive rows per fragment
    constexpr int B1 = 32 * BK * 2, B2 = (SWIGLU ? 128 : 64) * BK * 2, B3 = (SWIGLU ? 160 : 96) * BK * 2;

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
    const int lrow = lane / CH, lslot = lane % CH;

    // LDS byte address of this lane's first A and B fragment (stage 0, K
    // chunk 0) and the byte offset of its chunk in each 16-deep K sub-step:
    // lane l reads row l % 32 of each 32-row fragment at 16-byte chunk
    // 2 kk + l / 32, stored at chunk position (2 kk + l / 32) ^ swz(row).
    // Fragments start at multiples of 32 rows, so swz(row) depends only on l
    // and, for the row ^ (row / 8) permutation, on the fragment's parity.
    const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void*)&lds[0][0][0];
    constexpr uint32_t kStageBytes = 2 * STAGE_ELEMS * 2;
    // LDS rows this wave's loads fill: wid * 64 .. +63 of each operand
    const uint32_t lds_wave = __builtin_amdgcn_readfirstlane(lds_base + (uint32_t)(wid * 64 * BK * 2));
    const uint32_t a_rd = lds_base + (uint32_t)((wm * 128 + (lane & 31)) * BK * 2);
    const uint32_t b_rd = lds_base + (uint32_t)(STAGE_ELEMS * 2 + (SWIGLU ? wn * 64 : wn * 128) * BK * 2 +
                                                (lane & 31) * BK * 2);
    uint32_t koff[4][2];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int par = 0; par < 2; ++par)
            koff[kk][par] = (uint32_t)(((2 * kk + (lane >> 5)) ^ swz<SWZ>(par * 32 + (lane & 31))) << 4);
    // State of the unit in flight, set by `setup`: its tile, K stages
    // [kb, ke), partial-sum slot (-1: whole tile), load offsets and bases.
    int kb = 0, ke = 0, slot = -1, row0 = 0, row_end = 0, a_end = 0, nt = 0;
    bool valid = false;
    uint32_t aoff[LOADS], boff[LOADS];
    const char* abase = (const char*)p.A;
    const char* bbase = (const char*)p.B;
#define GG_LOAD_A(kt, stage, i)                                                                          \
    dma_lds16(lds_wave + (uint32_t)(stage) * kStageBytes + (i) * RPL * BK * 2, aoff[i], abase + (size_t)(kt) * (BK * 2))
#define GG_LOAD_B(kt, stage, i)                                                                          \
    dma_lds16(lds_wave + (uint32_t)(stage) * kStageBytes + STAGE_ELEMS * 2 + (i) * RPL * BK * 2, boff[i],         \
              bbase + (size_t)(kt) * (BK * 2))
#define GG_ISSUE(kt, stage)                                                                              \
    _Pragma("unroll") for (int i = 0; i < LOADS; ++i) {                                                  \
        GG_LOAD_A(kt, stage, i);                                                                         \
        GG_LOAD_B(kt, stage, i);                                                                         \
    }
// Wait until every LDS read issued so far has landed; the fragment registers
// are tied to the wait so no MFMA that uses them moves above it.
#define GG_WAIT_FRAGS(FA, FB)                                                                            \
    __asm__ volatile("s_waitcnt lgkmcnt(0)"                                                              \
                     : "+v"(FA[0]), "+v"(FA[1]), "+v"(FA[2]), "+v"(FA[3]), "+v"(FB[0]), "+v"(FB[1]),     \
                       "+v"(FB[2]), "+v"(FB[3])::"memory")
#define GG_MFMA(FA, FB, mi, ni)                                                                          \
    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(FA[mi], FB[ni], acc[mi][ni], 0, 0, 0)
// The 8 fragments of one K sub-step: A fragment mi at mi * 32 rows, B
// fragment ni at B1..B3 bytes past fragment 0; AD/BD[par] are the lane's
// addresses for fragments of parity par (the chunk permutation differs).
#define GG_RD_A(GA, AD, mi) GA[mi] = lds_frag<(mi) * 32 * BK * 2>(AD[(mi) & 1])
#define GG_RD_B(GB, BD, ni) GB[ni] = lds_frag<(ni) == 0 ? 0 : (ni) == 1 ? B1 : (ni) == 2 ? B2 : B3>(BD[(ni) & 1])
#define GG_SB __builtin_amdgcn_sched_barrier(0)
// One MFMA of a K sub-step, preceded by PRE (a load of a later stage, or
// nothing) and followed by RD (one fragment read of the next sub-step, or
// nothing); sched_barrier pins the order, so the matrix core has its next
// MFMA ready while the loads and reads are in flight.
#define GG_STEP(FA, FB, mi, ni, PRE, RD)                                                                 \
    PRE;                                                                                                 \
    GG_MFMA(FA, FB, mi, ni);                                                                             \
    RD;                                                                                                  \
    GG_SB;
// One K sub-step: 16 MFMAs on FA/FB; the 8 fragment reads of the next
// sub-step into GA/GB (addresses AD/BD) follow the first 8 of them, and
// L0..L7 (loads of a later stage, or nothing) precede every other MFMA: one
// 1 KiB load per two MFMAs per wave is what the CU's address unit sustains
// (about one such load per 16 cycles for the four wavefronts together).
#define GG_SUBSTEP_X(FA, FB, GA, GB, AD, BD, L0, L1, L2, L3, L4, L5, L6, L7)                             \
    GG_WAIT_FRAGS(FA, FB);                                                                               \
    GG_SB;                                                                                               \
    GG_STEP(FA, FB, 0, 0, L0, GG_RD_A(GA, AD, 0))                                                        \
    GG_STEP(FA, FB, 0, 1, (void)0, GG_RD_A(GA, AD, 1))                                                   \
    GG_STEP(FA, FB, 0, 2, L1, GG_RD_A(GA, AD, 2))                                                        \
    GG_STEP(FA, FB, 0, 3, (void)0, GG_RD_A(GA, AD, 3))                                                   \
    GG_STEP(FA, FB, 1, 0, L2, GG_RD_B(GB, BD, 0))                                                        \
    GG_STEP(FA, FB, 1, 1, (void)0, GG_RD_B(GB, BD, 1))                                                   \
    GG_STEP(FA, FB, 1, 2, L3, GG_RD_B(GB, BD, 2))                                                        \
    GG_STEP(FA, FB, 1, 3, (void)0, GG_RD_B(GB, BD, 3))                                                   \
    GG_STEP(FA, FB, 2, 0, L4, (void)0)                                                                   \
    GG_STEP(FA, FB, 2, 1, (void)0, (void)0)                                                              \
    GG_STEP(FA, FB, 2, 2, L5, (void)0)                                                                   \
    GG_STEP(FA, FB, 2, 3, (void)0, (void)0)                                                              \
    GG_STEP(FA, FB, 3, 0, L6, (void)0)                                                                   \
    GG_STEP(FA, FB, 3, 1, (void)0, (void)0)                                                              \
    GG_STEP(FA, FB, 3, 2, L7, (void)0)                                                                   \
    GG_STEP(FA, FB, 3, 3, (void)0, (void)0)
#define GG_N_ (void)0
#define GG_SUBSTEP(FA, FB, GA, GB, AD, BD)                                                               \
    GG_SUBSTEP_X(FA, FB, GA, GB, AD, BD, GG_N_, GG_N_, GG_N_, GG_N_, GG_N_, GG_N_, GG_N_, GG_N_)
// ... with the 8 A (B) loads of stage LKT into stage buffer LST
#define GG_SUBSTEP_LA(FA, FB, GA, GB, AD, BD, LKT, LST)                                                  \
    GG_SUBSTEP_X(FA, FB, GA, GB, AD, BD, GG_LOAD_A(LKT, LST, 0), GG_LOAD_A(LKT, LST, 1),                 \
                 GG_LOAD_A(LKT, LST, 2), GG_LOAD_A(LKT, LST, 3), GG_LOAD_A(LKT, LST, 4),                 \
                 GG_LOAD_A(LKT, LST, 5), GG_LOAD_A(LKT, LST, 6), GG_LOAD_A(LKT, LST, 7))
#define GG_SUBSTEP_LB(FA, FB, GA, GB, AD, BD, LKT, LST)                                                  \
    GG_SUBSTEP_X(FA, FB, GA, GB, AD, BD, GG_LOAD_B(LKT, LST, 0), GG_LOAD_B(LKT, LST, 1),                 \
                 GG_LOAD_B(LKT, LST, 2), GG_LOAD_B(LKT, LST, 3), GG_LOAD_B(LKT, LST, 4),                 \
                 GG_LOAD_B(LKT, LST, 5), GG_LOAD_B(LKT, LST, 6), GG_LOAD_B(LKT, LST, 7))

    // Decode unit u (from `take`), compute its tile's addressing and issue
    // the loads of its first stage and the A half of its second (stage
    // buffers 0 and 1).  Called right after the
    // previous unit's K loop, so these loads are in flight while that unit's
    // epilogue runs.  A wave's loads land in issue order, after the previous
    // unit's last (repeated) loads of the same rows.
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
        // uniform tile bases: 32-bit, so the loads take few registers.
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int r = wid * 64 + i * RPL + lrow;  // tile row 0..255
            const int chunk = lslot ^ swz<SWZ>(r);
            const int ar = min(row0 + r, a_end - 1);
            aoff[i] = p.src_map ? (uint32_t)(((size_t)(p.src_map[ar] / p.gk) * K + chunk * 8) * 2)
                                : (uint32_t)(((size_t)(ar - row0) * K + chunk * 8) * 2);
            int br;
            if (SWIGLU) {
                const int f = min(nt * 128 + out_col_swiglu(r & 127), p.n_out - 1);
                br = r < 128 ? f : p.n_out + f;
            } else {
                br = min(nt * kTile + out_col(r), p.n_out - 1);
            }
            boff[i] = (uint32_t)(((size_t)(br - brow0) * K + chunk * 8) * 2);
        }
        abase = p.src_map ? (const char*)p.A : (const char*)(p.A + (size_t)row0 * K);
        bbase = (const char*)(p.B + ((size_t)e * p.b_rows + brow0) * K);
        GG_SB;
        GG_ISSUE(kb, 0);
#pragma unroll
        for (int i = 0; i < LOADS; ++i) GG_LOAD_A(min(kb + 1, ke - 1), 1, i);
        GG_SB;
    };

    setup(unit);
    while (unit >= 0) {
        // Two LDS stages, software-pipelined across the stage boundary.  A stage
        // is four 16-deep K sub-steps of 16 MFMAs each; the fragments of
        // sub-step j+1 are read from LDS while the MFMAs of sub-step j issue.
        // The one barrier per stage sits before the last sub-step: by then
        // this wave has read all of stage kt and its loads of stage kt+1 have
        // landed; once every wave is past it the buffer of stage kt is free.
        // The loads of stage kt+2 go into it, the A half during the last
        // sub-step of stage kt and the B half during the first sub-step of
        // stage kt+1 (so the address unit is never oversubscribed).  Loads
        // past the end of K repeat the last stage into the free buffer, so
        // the loop has no branch.  (An L2 prefetch of later stages, one
        // 4-byte load per row, cost more address-unit time than it saved.)
        bf16x8 fa0[4], fb0[4], fa1[4], fb1[4];
        // the unit's first stage landed everywhere; the previous unit's stores retired
        __asm__ volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        GG_SB;
        if (tid == 0) {  // publish the next unit, take a ticket for the one after
            const int nu = take(tick);
            s_unit = nu;
            tick = nu >= 0 ? ticket() : -1;
        }
        f32x16 acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
        {
            const uint32_t ad[2] = {a_rd + koff[0][0], a_rd + koff[0][1]};
            const uint32_t bd[2] = {b_rd + koff[0][0], b_rd + koff[0][1]};
            GG_RD_A(fa0, ad, 0);
            GG_RD_A(fa0, ad, 1);
            GG_RD_A(fa0, ad, 2);
            GG_RD_A(fa0, ad, 3);
            GG_RD_B(fb0, bd, 0);
            GG_RD_B(fb0, bd, 1);
            GG_RD_B(fb0, bd, 2);
            GG_RD_B(fb0, bd, 3);
        }
        for (int kt = kb; kt < ke; ++kt) {
            const int st = (kt - kb) & 1;
            const uint32_t so = (uint32_t)st * kStageBytes;
            GG_SB;
            {
                const uint32_t ad[2] = {a_rd + so + koff[1][0], a_rd + so + koff[1][1]};
                const uint32_t bd[2] = {b_rd + so + koff[1][0], b_rd + so + koff[1][1]};
                GG_SUBSTEP_LB(fa0, fb0, fa1, fb1, ad, bd, min(kt + 1, ke - 1), st ^ 1)
            }
            {
                const uint32_t ad[2] = {a_rd + so + koff[2][0], a_rd + so + koff[2][1]};
                const uint32_t bd[2] = {b_rd + so + koff[2][0], b_rd + so + koff[2][1]};
                GG_SUBSTEP(fa1, fb1, fa0, fb0, ad, bd)
            }
            {
                const uint32_t ad[2] = {a_rd + so + koff[3][0], a_rd + so + koff[3][1]};
                const uint32_t bd[2] = {b_rd + so + koff[3][0], b_rd + so + koff[3][1]};
                GG_SUBSTEP(fa0, fb0, fa1, fb1, ad, bd)
            }
            // this wave has read all of stage kt and its loads of stage kt+1
            // landed; past the barrier, the same holds for every wave
            __asm__ volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
            GG_SB;
            {
                const uint32_t nso = so ^ kStageBytes;
                const uint32_t ad[2] = {a_rd + nso + koff[0][0], a_rd + nso + koff[0][1]};
                const uint32_t bd[2] = {b_rd + nso + koff[0][0], b_rd + nso + koff[0][1]};
                GG_SUBSTEP_LA(fa1, fb1, fa0, fb0, ad, bd, min(kt + 2, ke - 1), st)
            }
            // the next stage's first fragments landed (they had the last 8
            // MFMAs to do so); waiting here rather than at the top of the next
            // iteration leaves no LDS read in flight when the loop ends
            GG_WAIT_FRAGS(fa0, fb0);
        }
        GG_SB;
#undef GG_LOAD_A
#undef GG_LOAD_B
#undef GG_ISSUE
#undef GG_WAIT_FRAGS
#undef GG_MFMA
#undef GG_RD_A
#undef GG_RD_B
#undef GG_SB
#undef GG_STEP
#undef GG_SUBSTEP_X
#undef GG_N_
#undef GG_SUBSTEP
#undef GG_SUBSTEP_LA
#undef GG_SUBSTEP_LB


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
        // Epilogue straight from the accumulators (no LDS, so no barrier
        // before the next tile).  With the column order of the B rows above,
        // lane l holds, for each of its 16 rows of a 32-row block, adjacent
        // output columns in its four (SwiGLU: two) fragments: one 8-byte word
        // of four bf16 (SwiGLU: a 4-byte pair of h), so 32 lanes cover 256
        // (128) contiguous bytes of a row.  Opaque copies of the tile's first
        // row and of the lane index: the address arithmetic below then stays
        // after the K loop (it is not hoisted out of the tile loop, where it
        // would hold registers).
        int rbase = e_row0, ln = lane;
        __asm__ volatile("" : "+v"(rbase), "+v"(ln));
        const int lc = ln & 31;             // this lane's column group
        const int lr = 4 * (ln >> 5);       // this lane's first row in a 32-row block
        const int rlim = e_row_end - rbase;  // rows of the tile that exist
        const int alim = e_a_end - rbase;    // rows of the tile that are not padding (gather)
        // Store W[q] (type T) to row 8 (q / 4) + q % 4 past DST (LD elements
        // per row) for q = 0..15: the lane's rows of the 32-row block starting
        // at tile row RB0; rows are checked only when the block runs past the
        // group's end.
        // RW[q]: the routing weight of the lane's row 8 (q / 4) + q % 4 of
        // 32-row block MI (1 without weights); row i of the wave's band sits
        // in lane i / 2, as rwa (even i) or rwb (odd i).
#define GB_ROW_WEIGHTS(MI, W_)                                                                           \
    if constexpr ((EP & 1) != 0) {                                                                       \
        _Pragma("unroll") for (int q = 0; q < 16; ++q)                                                   \
            W_[q] = __shfl((q & 1) ? rwb : rwa, ((MI) * 32 + lr + 8 * (q >> 2) + (q & 3)) >> 1, 64);     \
    } else {                                                                                             \
        _Pragma("unroll") for (int q = 0; q < 16; ++q) W_[q] = 1.f;                                      \
    }
#define GB_STORE_ROWS(T, DST, LD, RB0, W)                                                                \
    if ((RB0) + 32 <= rlim) {                                                                            \
        _Pragma("unroll") for (int q = 0; q < 16; ++q)                                                   \
            *(T*)((DST) + (size_t)(8 * (q >> 2) + (q & 3)) * (LD)) = (W)[q];                             \
    } else {                                                                                             \
        _Pragma("unroll") for (int q = 0; q < 16; ++q)                                                   \
            if ((RB0) + lr + 8 * (q >> 2) + (q & 3) < rlim)                                              \
                *(T*)((DST) + (size_t)(8 * (q >> 2) + (q & 3)) * (LD)) = (W)[q];                         \
    }

        if (e_slot >= 0) {
            // a K part of a split tile: its float32 partial sums, all 256 x 256
            // (rows past the group's end and columns past the output width
            // included; the reduction skips them), in [row][column] order with
            // SwiGLU gate columns 0..127 and up columns 128..255
            float* const pb = p.part + (size_t)e_slot * kTile * kTile;
#define GB_EPI_PART(MI)                                                                                  \
    {                                                                                                    \
        const int rb0 = wm * 128 + (MI) * 32;                                                            \
        float* const prow = pb + (size_t)(rb0 + lr) * kTile;                                             \
        if (SWIGLU) {                                                                                    \
            float2 gw[16], uw[16];                                                                       \
            _Pragma("unroll") for (int q = 0; q < 16; ++q) {                                             \
                gw[q] = make_float2(agpr_read(acc[MI][0][q]), agpr_read(acc[MI][1][q]));                 \
                uw[q] = make_float2(agpr_read(acc[MI][2][q]), agpr_read(acc[MI][3][q]));                 \
            }                                                                                            \
            _Pragma("unroll") for (int q = 0; q < 16; ++q) {                                             \
                float* const d = prow + (size_t)(8 * (q >> 2) + (q & 3)) * kTile + wn * 64 + 2 * lc;     \
                *(float2*)d = gw[q];                                                                     \
                *(float2*)(d + 128) = uw[q];                                                             \
            }                                                                                            \
        } else {                                                                                         \
            float4 w[16];                                                                                \
            _Pragma("unroll") for (int q = 0; q < 16; ++q)                                               \
                w[q] = make_float4(agpr_read(acc[MI][0][q]), agpr_read(acc[MI][1][q]),                   \
                                   agpr_read(acc[MI][2][q]), agpr_read(acc[MI][3][q]));                  \
            _Pragma("unroll") for (int q = 0; q < 16; ++q)                                               \
                *(float4*)(prow + (size_t)(8 * (q >> 2) + (q & 3)) * kTile + wn * 128 + 4 * lc) = w[q];  \
        }                                                                                                \
    }                                                                                                    \
    __builtin_amdgcn_sched_barrier(0);
            GB_EPI_PART(0) GB_EPI_PART(1) GB_EPI_PART(2) GB_EPI_PART(3)
#undef GB_EPI_PART
        } else if (SWIGLU) {
            uint16_t* const cbase = p.C + (size_t)rbase * p.n_out;
            uint16_t* const sbase = p.stash ? p.stash + (size_t)rbase * 2 * p.n_out : nullptr;
            const int f = e_nt * 128 + wn * 64 + 2 * lc;  // this lane's h columns f, f + 1
#define GB_EPI_SW(MI)                                                                                    \
    {                                                                                                    \
        const int rb0 = wm * 128 + (MI) * 32;                                                            \
        uint32_t hw[16];                                                                                 \
        float rw[16];                                                                                    \
        GB_ROW_WEIGHTS(MI, rw)                                                                           \
        _Pragma("unroll") for (int q = 0; q < 16; ++q) {                                                 \
            float g0 = agpr_read(acc[MI][0][q]), g1 = agpr_read(acc[MI][1][q]);                          \
            float u0 = agpr_read(acc[MI][2][q]), u1 = agpr_read(acc[MI][3][q]);                          \
            if constexpr ((EP & 2) != 0) {                                                               \
                g0 = fminf(g0, p.lim);                                                                   \
                g1 = fminf(g1, p.lim);                                                                   \
                u0 = fminf(fmaxf(u0, -p.lim), p.lim);                                                    \
                u1 = fminf(fmaxf(u1, -p.lim), p.lim);                                                    \
            }                                                                                            \
            hw[q] = pack_bf16x2(silu(g0) * u0 * rw[q], silu(g1) * u1 * rw[q]);                           \
            if (rb0 + lr + 8 * (q >> 2) + (q & 3) >= alim) hw[q] = 0; /* gather: padding rows */         \
        }                                                                                                \
        if (f < p.n_out) {                                                                               \
            uint16_t* const dst = cbase + (size_t)(rb0 + lr) * p.n_out + f;                              \
            GB_STORE_ROWS(uint32_t, dst, p.n_out, rb0, hw)                                               \
            if (sbase) {                                                                                 \
                uint32_t gw[16], uw[16];                                                                 \
                _Pragma("unroll") for (int q = 0; q < 16; ++q) {                                         \
                    gw[q] = pack_bf16x2(agpr_read(acc[MI][0][q]), agpr_read(acc[MI][1][q]));             \
                    uw[q] = pack_bf16x2(agpr_read(acc[MI][2][q]), agpr_read(acc[MI][3][q]));             \
                }                                                                                        \
                uint16_t* const gd = sbase + (size_t)(rb0 + lr) * 2 * p.n_out + f;                       \
                GB_STORE_ROWS(uint32_t, gd, 2 * p.n_out, rb0, gw)                                        \
                uint16_t* const ud = gd + p.n_out;                                                       \
                GB_STORE_ROWS(uint32_t, ud, 2 * p.n_out, rb0, uw)                                        \
            }                                                                                            \
        }                                                                                                \
    }                                                                                                    \
    __builtin_amdgcn_sched_barrier(0);
            GB_EPI_SW(0) GB_EPI_SW(1) GB_EPI_SW(2) GB_EPI_SW(3)
#undef GB_EPI_SW
        } else {
            uint16_t* const cbase = p.C + (size_t)rbase * p.n_out;
            const int n = e_nt * kTile + wn * 128 + 4 * lc;  // this lane's columns n .. n + 3
#define GB_EPI_DN(MI)                                                                                    \
    {                                                                                                    \
        const int rb0 = wm * 128 + (MI) * 32;                                                            \
        uint2 w[16];                                                                                     \
        float rw[16];                                                                                    \
        GB_ROW_WEIGHTS(MI, rw)                                                                           \
        _Pragma("unroll") for (int q = 0; q < 16; ++q)                                                   \
            w[q] = make_uint2(pack_bf16x2(agpr_read(acc[MI][0][q]) * rw[q], agpr_read(acc[MI][1][q]) * rw[q]), \
                              pack_bf16x2(agpr_read(acc[MI][2][q]) * rw[q], agpr_read(acc[MI][3][q]) * rw[q])); \
        if (n < p.n_out) {                                                                               \
            uint16_t* const dst = cbase + (size_t)(rb0 + lr) * p.n_out + n;                              \
            GB_STORE_ROWS(uint2, dst, p.n_out, rb0, w)                                                   \
        }                                                                                                \
    }                                                                                                    \
    __builtin_amdgcn_sched_barrier(0);
            GB_EPI_DN(0) GB_EPI_DN(1) GB_EPI_DN(2) GB_EPI_DN(3)
#undef GB_EPI_DN
        }
#undef GB_STORE_ROWS
#undef GB_ROW_WEIGHTS
        }  // valid
        unit = next_unit;
    }
}

}  // namespace gemm
}  // namespace moe
