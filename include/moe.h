/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE FFN hot path.
 *
 * The path (one GPU's share of a Mixture-of-Experts FFN block):
 *   route -> permute -> grouped gate/up GEMM + SwiGLU -> grouped down GEMM
 *   -> top-k weighted combine, and the FFN backward.
 *
 * Sources (web pages, cited by title and section):
 *   [TE-EP]  "[JAX] Expert Parallelism: JAX primitives + VJPs"
 *            (TransformerEngine PR #3036): Summary (dispatch/combine return the
 *            per-expert token counts; routing state is cached for the backward;
 *            the calls are CUDA-graph capturable) and its squashed commit
 *            messages (fp32 router, sum + 1e-20 normalisation, expert-major
 *            zero-padded layout, device token counts as grouped-GEMM group
 *            sizes, zero weight gradients for 0-token experts, d_x in x's dtype).
 *   [CUDNN]  "Add MoE + expert-parallel Python API surface, PyTorch reference,
 *            and tests" (cudnn-frontend PR #389): Summary (routing with -1 as
 *            a dropped route, local SwiGLU experts silu(gate)*up, per-top-k
 *            combine, backward from a saved pre-SwiGLU stash) and the review
 *            comments quoting MoeEp.__call__ (logical shapes activation (T,H),
 *            fc1 (E,H,2I), fc2 (E,I,H), topk (T,K)), backward and
 *            BlockScaledTensor (MXFP8 block 32).
 *   [ISSUE]  "MoE training optimization" (TransformerEngine issue #2438):
 *            sync-free MoE, all problem sizes supplied from device buffers.
 *   [BLOCK]  "[Draft][JAX] MoE block optimization" (TransformerEngine
 *            PR #3638), Diagram: route, dispatch, fused grouped GEMM + SwiGLU,
 *            down projection, combine.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Memory.  Every pointer argument except `cfg` is device memory (HBM of the
 *   current HIP device) allocated and owned by the caller; the library never
 *   allocates, frees or keeps a pointer after returning.  Scratch space comes
 *   only from the caller's workspace `ws` of `ws_bytes` bytes
 *   (moe_workspace_size for the forward calls, moe_backward_workspace_size for
 *   the backward GEMMs).  Every pointer is 16-byte aligned (hipMalloc and
 *   torch give 256): a required pointer that is NULL or misaligned, or a
 *   misaligned optional one, is MOE_ERR_INVALID_ARG.  Pointers are not checked
 *   for residency.
 * - Streams.  `stream` is a hipStream_t (NULL = the null stream).  Every call
 *   only enqueues kernels on it and returns: no host synchronisation, no
 *   device-to-host copy, no host read of counts or offsets ([ISSUE]), so the
 *   calls are safe under HIP graph capture.  Data-dependent sizes (per-expert
 *   counts and offsets) live in device buffers; grids are sized from host-known
 *   bounds (T, k, E, align).
 * - Errors.  A call returns MOE_OK or an error status; moe_last_error() then
 *   holds a message (per thread).  Every host-side check (null required
 *   pointers, sizes, dtype combinations, workspace size) runs before the
 *   first launch, the fused calls included, so MOE_ERR_INVALID_ARG,
 *   MOE_ERR_UNSUPPORTED and MOE_ERR_WORKSPACE mean nothing was enqueued.
 *   MOE_ERR_HIP reports a failed kernel launch (the kernels of the same call
 *   enqueued before it stay enqueued).  Expert ids outside [-1, E) in a
 *   routing table can only be seen on the device: such routes are dropped and
 *   counted in the optional device counter `err`.
 * - Layouts (row-major, innermost last).  x [T,H]; logits [T,E] float32;
 *   idx [T,k] int32; w [T,k] float32.  Expert weights are stored with the
 *   contraction dimension contiguous: w1 [E][2F][H] holds the logical fc1
 *   (E,H,2F) transposed, rows [0,F) = gate columns, rows [F,2F) = up columns;
 *   w2 [E][H][F] holds the logical fc2 (E,F,H) transposed.  Permuted
 *   activations Xp [R_cap,H], h [R_cap,F], Yp [R_cap,H] are expert-major
 *   ([TE-EP]): expert e owns rows [offsets[e], offsets[e+1]), the first
 *   counts[e] of them real routes in ascending token order, the rest zero
 *   padding up to a multiple of `align`; rows from offsets[E] to R_cap are an
 *   unused tail that no call reads or writes.  R_cap = T*k + E*(align-1).
 * - Dtypes.  cfg->dtype is the storage of x, the weights, Xp and h:
 *   MOE_F32, MOE_BF16 or MOE_MXFP8 (OCP E4M3 codes, one byte each, plus one
 *   E8M0 scale byte per 32 consecutive elements of the contiguous dimension:
 *   x_scale [T,H/32], w1_scale [E][2F][H/32], w2_scale [E][H][F/32],
 *   h_scale [R_cap,F/32]).  MOE_MXFP4 (the MX analogue of [ISSUE]'s and
 *   [CUDNN]'s NVFP4 recipe, native to CDNA4's scaled matrix cores): OCP E2M1
 *   codes (1 sign, 2 exponent bits, 1 mantissa bit; magnitudes 0, 0.5, 1, 1.5,
 *   2, 3, 4, 6) packed two per byte, element 2i in the low 4 bits of byte i, so
 *   a row of n elements is n/2 bytes (x [T,H/2], w1 [E][2F][H/2], w2
 *   [E][H][F/2], Xp [R_cap,H/2], h [R_cap,F/2]), with the same E8M0 scale
 *   arrays as MXFP8; H and F must be multiples of 512.  Yp and y (and all
 *   activation gradients) are float32 when dtype is MOE_F32 and bfloat16
 *   otherwise ([TE-EP]: the output keeps x's dtype; MX layers return bfloat16
 *   per [CUDNN]).  Every GEMM
 *   accumulates in float32 and rounds once when it stores.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1, /* null pointer, bad size or enum value          */
    MOE_ERR_UNSUPPORTED = 2, /* valid but not built: e.g. H % 64 != 0          */
    MOE_ERR_WORKSPACE = 3,   /* ws NULL or ws_bytes below the call's need      */
    MOE_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed    */
} moe_status;

typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1, MOE_MXFP8 = 2, MOE_MXFP4 = 3 } moe_dtype;
typedef enum moe_score { MOE_SOFTMAX = 0, MOE_SIGMOID = 1 } moe_score;
/* Where moe_forward applies the routing weights ([CUDNN] Summary: the router
 * weight in the FC1 or the FC2 epilogue; [TE-EP] commits: the weights may be
 * applied before the combine).  In exact arithmetic the three give the same
 * y; they differ in where the weight meets a rounding.
 *   MOE_WEIGHT_AT_COMBINE: y[t] = sum_j w[t,j] Yp[row]          (default)
 *   MOE_WEIGHT_AT_FC1:     h[row] = store(w[t,j] silu(g) u), y[t] = sum_j Yp[row]
 *   MOE_WEIGHT_AT_FC2:     Yp[row] = store(w[t,j] h W2^T),  y[t] = sum_j Yp[row]
 * The backward calls (moe_combine_bwd, moe_backward, moe_route_bwd) are built
 * for MOE_WEIGHT_AT_COMBINE and return MOE_ERR_UNSUPPORTED otherwise. */
typedef enum moe_weight_site { MOE_WEIGHT_AT_COMBINE = 0, MOE_WEIGHT_AT_FC1 = 1, MOE_WEIGHT_AT_FC2 = 2 } moe_weight_site;

typedef struct moe_config {
    int32_t T;      /* tokens (>= 0)                                         */
    int32_t H;      /* hidden size (multiple of 128; of 512 for MXFP4)       */
    int32_t F;      /* per-expert FFN width (multiple of 64; of 128 for MXFP8;
                       of 512 for MXFP4)                                     */
    int32_t E;      /* experts (1..1024)                                     */
    int32_t k;      /* routes per token (1..min(E, 64))                      */
    int32_t align;  /* per-expert row alignment (>= 1)                       */
    int32_t score;  /* moe_score                                             */
    int32_t renorm; /* softmax: 1 = renormalise over the k selected;
                       sigmoid: always normalised over the k selected        */
    int32_t dtype;  /* moe_dtype of x / weights / Xp / h                     */
    int32_t weight_site; /* moe_weight_site: where moe_forward applies w     */
    float swiglu_limit;  /* optional SwiGLU clamp ([CUDNN] Summary: optional
                            DeepSeek-style clamp; no bounds on the pages):
                            L > 0: h = silu(min(g, L)) * clamp(u, -L, L) in
                            every gate/up GEMM, and the backward passes the
                            gradient only where the bound is not exceeded
                            (bounds included); 0: no clamp.  The stash keeps
                            the unclamped g and u.  Must be finite, >= 0.    */
} moe_config;

/* Rows of the permuted buffers: T*k + E*(align-1).  Host only. */
int64_t moe_rows_capacity(const moe_config* cfg);

/* Bytes of scratch moe_permute, the grouped GEMMs and moe_forward need for
 * this config (0 is possible; for bf16 storage about 64 MiB: the GEMMs'
 * work-queue counters and the float32 partial sums of tiles cut along K).
 * Host only; no device access. */
size_t moe_workspace_size(const moe_config* cfg);

/* Bytes of scratch moe_grouped_down_bwd, moe_grouped_swiglu_bwd and
 * moe_backward need (0 is possible; at most about 1 GiB).  The weight
 * gradients cut an expert with many rows into row ranges computed in
 * parallel; their float32 partial sums live here and are added in row order,
 * so the result does not depend on scheduling.  Host only. */
size_t moe_backward_workspace_size(const moe_config* cfg);

/* Step 1, routing ([TE-EP] fp32 router with both score functions and the
 * sum + 1e-20 normalisation; [CUDNN] routing).  For each token t the k largest
 * logits are selected, in descending order, equal logits going to the lower
 * expert index; idx[t,j] is the j-th selected expert.  Weights:
 *   softmax: p = exp(l - max_e l) / sum_e exp(l_e - max_e l) over all E;
 *            w = p, or p / (sum of the k selected p + 1e-20) when renorm;
 *   sigmoid: s = 1 / (1 + exp(-l)); w = s / (sum of the k selected s + 1e-20).
 * Expert bias ([TE-EP] router commits: optional expert routing bias; a zero
 * bias behaves as none): bias (optional, NULL for none) [E] f32 shifts only
 * the selection, which then ranks the key fl32(l[e] + bias[e]) (ties again to
 * the lower index); the weights above are still formed from the unbiased
 * logits of the chosen experts.  A zero bias gives the same bytes as NULL.
 * The bias gets no gradient (the choice is piecewise constant); moe_route_bwd
 * works unchanged on a biased idx.
 * logits [T,E] f32 (finite) -> idx [T,k] i32, w [T,k] f32. */
moe_status moe_route(const moe_config* cfg, const float* logits, const float* bias, int32_t* idx, float* w,
                     void* stream);

/* Step 2, grouping and permutation ([TE-EP] expert-major layout with per-expert
 * zero padding; device token counts; [ISSUE] no device-to-host sync;
 * [CUDNN] -1 = dropped route).  From idx [T,k]:
 *   counts[e]      = routes to expert e                           [E]
 *   offsets[e]     = sum_{e'<e} align*ceil(counts[e']/align)      [E+1]
 *   row_map[t*k+j] = row of route (t,j) in Xp, -1 if dropped      [T,k]
 *   src_map[row]   = t*k+j for real rows, -1 for padding rows and
 *                    the tail [offsets[E], R_cap)                 [R_cap]
 *   Xp[row_map[t,j]] = x[t] byte for byte; padding rows zero     [R_cap,H]
 * Within an expert, routes are in ascending (t, j) order, so every output is
 * deterministic.  MXFP8: x_scale rows travel with x into xp_scale (both NULL
 * otherwise).  err (optional, may be NULL) is incremented once per id
 * outside [-1, E).  xp NULL: the grouping only (counts .. src_map), for the
 * gather form of the gate/up GEMM below; x, x_scale, xp_scale are then not
 * read.  ws: moe_workspace_size(cfg) bytes. */
moe_status moe_permute(const moe_config* cfg, const void* x, const uint8_t* x_scale, const int32_t* idx, void* xp,
                       uint8_t* xp_scale, int32_t* counts, int32_t* offsets, int32_t* row_map, int32_t* src_map,
                       int32_t* err, void* ws, size_t ws_bytes, void* stream);

/* Step 3, grouped gate/up GEMM fused with SwiGLU ([BLOCK] fused grouped GEMM
 * and SwiGLU; [CUDNN] silu(gate) * up).  For every expert e and every row r in
 * [offsets[e], offsets[e+1]):
 *   g = Xp[r] . w1[e][f][:],  u = Xp[r] . w1[e][F+f][:]   (float32 sums)
 *   h[r][f] = silu(g) * u,  silu(g) = g / (1 + exp(-g)), stored in cfg->dtype
 *   (MXFP8: quantised per 32 columns with the OCP MX rule into h / h_scale).
 * Group sizes are read from `offsets` on the device; empty experts cost no
 * tiles.  gu_stash (optional, [R_cap,2F] in the output dtype) receives g in
 * columns [0,F) and u in [F,2F) for the backward ([CUDNN] fc1 stash).
 * xp_scale / w1_scale / h_scale: MXFP8 only, NULL otherwise.
 * ws: moe_workspace_size(cfg) bytes (the same scratch moe_permute takes; the
 * bf16 and MXFP8 GEMMs keep their work-queue counters there, the bf16 ones
 * also the partial sums of tiles cut along K, so calls sharing one workspace
 * must not overlap). */
moe_status moe_grouped_swiglu_gemm(const moe_config* cfg, const void* xp, const uint8_t* xp_scale, const void* w1,
                                   const uint8_t* w1_scale, const int32_t* offsets, void* h, uint8_t* h_scale,
                                   void* gu_stash, void* ws, size_t ws_bytes, void* stream);

/* Step 3 with step 2's permutation folded into the operand loads, so that
 * no Xp is materialised ([BLOCK] Diagram shows dispatch and the grouped GEMM
 * as two steps; this variant computes their composition): as
 * moe_grouped_swiglu_gemm, with row r of the grouped operand read as
 * x[src_map[r] / k] (the token routed to row r) for the first counts[e] rows
 * of expert e, and the padding rows of its group computed as zero rows.  h
 * (+ h_scale) equals, bit for bit, what moe_grouped_swiglu_gemm writes from
 * the Xp of moe_permute.  x [T,H] (+ x_scale [T,H/32] for MXFP8); src_map,
 * counts, offsets from moe_permute (which may skip Xp: xp NULL).  No stash
 * (a training forward keeps Xp for the weight gradient).  Needs
 * T*H*element size < 4 GiB (MOE_ERR_UNSUPPORTED otherwise).  ws: as for
 * moe_grouped_swiglu_gemm. */
moe_status moe_grouped_swiglu_gemm_gather(const moe_config* cfg, const void* x, const uint8_t* x_scale,
                                          const int32_t* src_map, const int32_t* counts, const void* w1,
                                          const uint8_t* w1_scale, const int32_t* offsets, void* h, uint8_t* h_scale,
                                          void* ws, size_t ws_bytes, void* stream);

/* Step 3 with the routing weight in its epilogue ([CUDNN] Summary: router
 * weight in the FC1 epilogue): as moe_grouped_swiglu_gemm, with
 *   h[r][f] = store( w[src_map[r]] * silu(g) * u )
 * (MXFP8: the weighted values are quantised); padding rows (src_map -1) get
 * weight 0.  src_map [R_cap] and w [T*k] from moe_permute / moe_route.  No
 * stash.  The per-row weights are written into ws first (part of
 * moe_workspace_size).  Combine such rows with moe_combine(w = NULL). */
moe_status moe_grouped_swiglu_gemm_weighted(const moe_config* cfg, const void* xp, const uint8_t* xp_scale,
                                            const void* w1, const uint8_t* w1_scale, const int32_t* offsets,
                                            const int32_t* src_map, const float* w, void* h, uint8_t* h_scale,
                                            void* ws, size_t ws_bytes, void* stream);

/* Step 4, grouped down GEMM ([BLOCK] down projection).  For every expert e
 * and row r in [offsets[e], offsets[e+1]):
 *   Yp[r][o] = h[r] . w2[e][o][:]   (float32 sum, stored in the output dtype).
 * h_scale / w2_scale: MXFP8 only.  ws: as for moe_grouped_swiglu_gemm. */
moe_status moe_grouped_down_gemm(const moe_config* cfg, const void* h, const uint8_t* h_scale, const void* w2,
                                 const uint8_t* w2_scale, const int32_t* offsets, void* yp, void* ws, size_t ws_bytes,
                                 void* stream);

/* Step 4 with the routing weight in its epilogue ([CUDNN] Summary: router
 * weight in the FC2 epilogue): as moe_grouped_down_gemm, with
 *   Yp[r][o] = store( w[src_map[r]] * (h[r] . w2[e][o][:]) )
 * (the float32 sum times the weight, rounded once); padding rows get weight
 * 0.  src_map, w and ws as for moe_grouped_swiglu_gemm_weighted.  Combine
 * such rows with moe_combine(w = NULL). */
moe_status moe_grouped_down_gemm_weighted(const moe_config* cfg, const void* h, const uint8_t* h_scale,
                                          const void* w2, const uint8_t* w2_scale, const int32_t* offsets,
                                          const int32_t* src_map, const float* w, void* yp, void* ws,
                                          size_t ws_bytes, void* stream);

/* Step 5, top-k weighted combine ([CUDNN] per-top-k combine; [TE-EP] expert
 * outputs summed across the top-k).
 *   y[t] = round( sum_{j ascending, row_map[t,j] != -1} w[t,j] * Yp[row_map[t,j]] )
 * summed in float32 and rounded once to the output dtype.  Rows no route maps
 * are never read, so padding and the tail may hold anything.  w NULL: the
 * weights were applied in an expert epilogue, and the routes are summed
 * (y[t] = round(sum_j Yp[row_map[t,j]])). */
moe_status moe_combine(const moe_config* cfg, const void* yp, const int32_t* row_map, const float* w, void* y,
                       void* stream);

/* The whole forward in one call: moe_route (bias as there), moe_permute,
 * moe_grouped_swiglu_gemm, moe_grouped_down_gemm, moe_combine on one stream.
 * Every buffer is the caller's: the routing outputs (idx, w, counts, offsets,
 * row_map, src_map), the permuted activations xp (+ xp_scale), h (+ h_scale),
 * yp, the output y [T,H], and gu_stash (NULL unless the backward will run).
 * Buffers another call would read later (idx .. src_map, xp, h, gu_stash) are
 * the routing state and saved tensors of the backward ([TE-EP]: no second
 * routing pass in the backward).  xp NULL (with xp_scale NULL and gu_stash
 * NULL: inference): the permutation is fused into the gate/up GEMM
 * (moe_grouped_swiglu_gemm_gather) and Xp is never written; the outputs are
 * the same bit for bit.  cfg->weight_site picks where w is applied: in the
 * combine, or in the gate/up (FC1) or down (FC2) epilogue (both forms). */
moe_status moe_forward(const moe_config* cfg, const float* logits, const float* bias, const void* x,
                       const uint8_t* x_scale, const void* w1, const uint8_t* w1_scale, const void* w2,
                       const uint8_t* w2_scale, void* y,
                       int32_t* idx, float* w, int32_t* counts, int32_t* offsets, int32_t* row_map,
                       int32_t* src_map, void* xp, uint8_t* xp_scale, void* h, uint8_t* h_scale, void* yp,
                       void* gu_stash, int32_t* err, void* ws, size_t ws_bytes, void* stream);

/* moe_forward without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments (ws and ws_bytes dropped), same
 * kernels and the same results bit for bit.  Its scratch space is a static
 * device array of the library, 68 MiB on every device the library is loaded
 * on, held until the process ends; a config whose moe_workspace_size exceeds
 * 68 MiB returns MOE_ERR_WORKSPACE.  The call allocates nothing.  The array
 * is shared by every call on a device and keeps the last call's contents:
 * calls that overlap on one device (other streams, other host threads) race,
 * so the caller orders them. */
moe_status moe_forward_noalloc(const moe_config* cfg, const float* logits, const float* bias, const void* x,
                               const uint8_t* x_scale, const void* w1, const uint8_t* w1_scale, const void* w2,
                               const uint8_t* w2_scale, void* y, int32_t* idx, float* w, int32_t* counts, int32_t* offsets, int32_t* row_map,
                               int32_t* src_map, void* xp, uint8_t* xp_scale, void* h, uint8_t* h_scale, void* yp,
                               void* gu_stash, int32_t* err, void* stream);

/* ---------------------------------------------------------------------- */
/* Backward of the expert FFN and the combine.  Built for BF16 storage    */
/* with the routing weights applied in the combine: every call below except */
/* moe_route_bwd (which also takes F32 and MXFP8 layers) returns           */
/* MOE_ERR_UNSUPPORTED for F32 or MXFP8 configs or an epilogue weight site. */
/* [TE-EP]: weight gradients of experts with no rows are zero; d_x keeps x's */
/* dtype.  [CUDNN]: the backward re-dispatches the output gradient along the */
/* forward routes and recomputes SwiGLU from the saved stash.  The routing   */
/* weights are constants here; moe_route_bwd gives their gradient.           */
/* ---------------------------------------------------------------------- */

/* Routing backward ([TE-EP] router commits; [CUDNN] per-top-k combine): for
 * an upstream gradient dy of the combine's output y[t] = sum_j w[t,j] Yp[...],
 *   dw[t][j]      = sum_c dy[t][c] * Yp[row_map[t,j]][c]   (float32; 0 for a
 *                   dropped route, row -1)
 *   dlogits[t][e] = sum_j dw[t][j] * d w[t][j] / d logits[t][e]
 * through moe_route's normalisation (softmax over all E; softmax renormalised
 * over the k selected; sigmoid normalised over the k selected); the top-k
 * choice itself has no gradient, so with renormalisation or the sigmoid only
 * the selected experts' logits get a nonzero gradient.  dy [T,H] and yp
 * [R_cap,H] in the output dtype (bf16 for BF16 and MXFP8 storage, float for
 * F32); logits [T,E] float (moe_route's input); idx [T,k] and row_map [T,k]
 * from moe_route / moe_permute; dw (optional, NULL to skip) [T,k] float;
 * dlogits [T,E] float, every entry written. */
moe_status moe_route_bwd(const moe_config* cfg, const void* dy, const void* yp, const float* logits,
                         const int32_t* idx, const int32_t* row_map, float* dw, float* dlogits, void* stream);

/* dYp[row_map[t,j]] = round(w[t,j] * dy[t]) for every route (t,j) whose
 * row_map entry is a row in [0, R_cap); dYp[r] = 0 for every row r in
 * [0, offsets[E]) whose src_map entry is not a route index in [0, T*k) (the
 * padding rows).  row_map and src_map are the two directions of one
 * permutation, as moe_permute writes them.  dy [T,H], dyp [R_cap,H], output
 * dtype. */
moe_status moe_combine_bwd(const moe_config* cfg, const void* dy, const int32_t* row_map, const int32_t* src_map,
                           const int32_t* offsets, const float* w, void* dyp, void* stream);

/* Down-projection backward fused with the SwiGLU backward, per expert rows:
 *   dH[r][f] = sum_o dYp[r][o] * w2[e][o][f]
 *   with g, u from gu_stash: sig = 1/(1+exp(-g)),
 *   dgu[r][f] = round(dH * u * sig * (1 + g*(1-sig))), dgu[r][F+f] = round(dH * g * sig)
 *   dw2[e][o][f] = sum_{r of e, ascending} h[r][f] * dYp[r][o]   (float32,
 *   exactly 0 for an expert with no rows).
 * dgu [R_cap,2F] output dtype; dw2 [E][H][F] float32 (the w2 layout).
 * ws: moe_backward_workspace_size(cfg) bytes. */
moe_status moe_grouped_down_bwd(const moe_config* cfg, const void* dyp, const void* w2, const void* h,
                                const void* gu_stash, const int32_t* offsets, void* dgu, float* dw2, void* ws,
                                size_t ws_bytes, void* stream);

/* Gate/up-projection backward, per expert rows:
 *   dXp[r][c] = round( sum_n dgu[r][n] * w1[e][n][c] )
 *   dw1[e][n][c] = sum_{r of e, ascending} dgu[r][n] * Xp[r][c]  (float32,
 *   exactly 0 for an expert with no rows).
 * dxp [R_cap,H] output dtype; dw1 [E][2F][H] float32 (the w1 layout).
 * ws: moe_backward_workspace_size(cfg) bytes. */
moe_status moe_grouped_swiglu_bwd(const moe_config* cfg, const void* dgu, const void* w1, const void* xp,
                                  const int32_t* offsets, void* dxp, float* dw1, void* ws, size_t ws_bytes,
                                  void* stream);

/* dx[t] = round( sum_{j ascending, row_map[t,j] != -1} dXp[row_map[t,j]] ),
 * summed in float32.  dx [T,H] in x's dtype. */
moe_status moe_permute_bwd(const moe_config* cfg, const void* dxp, const int32_t* row_map, void* dx, void* stream);

/* The whole backward in one call: moe_combine_bwd, moe_grouped_down_bwd,
 * moe_grouped_swiglu_bwd, moe_permute_bwd.  Inputs: dy, the routing state and
 * saved tensors of moe_forward (w, offsets, row_map, src_map, xp, h,
 * gu_stash) and the weights; outputs dx, dw1, dw2; dyp, dgu, dxp are the
 * caller's intermediate buffers.  ws: moe_backward_workspace_size(cfg) bytes. */
moe_status moe_backward(const moe_config* cfg, const void* dy, const float* w, const void* w1, const void* w2,
                        const int32_t* offsets, const int32_t* row_map, const int32_t* src_map, const void* xp,
                        const void* h, const void* gu_stash, void* dyp, void* dgu, void* dxp, void* dx, float* dw1,
                        float* dw2, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------- */
/* MXFP8 quantisation ([CUDNN] BlockScaledTensor, block 32 along the last   */
/* axis; [ISSUE] grouped MXFP8 quantisation), OCP MX v1.0 rule: per block of */
/* 32, shared exponent = floor(log2(max|v|)) - 8 clamped to [-127, 127]     */
/* (all-zero block -> code 0), elements v / 2^shared rounded to nearest even */
/* E4M3, saturating at +-448.  in [rows, cols] f32, cols % 32 == 0 ->       */
/* codes [rows, cols] u8, scales [rows, cols/32] u8 (E8M0).  Finite inputs.  */
/* ---------------------------------------------------------------------- */
moe_status moe_quantize_mxfp8(const float* in, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                              void* stream);

/* MXFP4 quantisation (the same OCP MX v1.0 rule with E2M1 elements): per block
 * of 32, shared exponent = floor(log2(max|v|)) - 2 clamped to [-127, 127]
 * (all-zero block -> code 0), elements v / 2^shared rounded to nearest even
 * E2M1, saturating at +-6; a value that rounds to zero keeps its sign (code
 * 8 for negative).  in [rows, cols] f32, cols % 32 == 0 -> codes [rows,
 * cols/2] u8 (element 2i in the low 4 bits of byte i), scales [rows, cols/32]
 * u8 (E8M0).  Finite inputs. */
moe_status moe_quantize_mxfp4(const float* in, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                              void* stream);

/* Message of the last failing call on this thread ("" if none). */
const char* moe_last_error(void);
/* Name of a status code. */
const char* moe_status_string(moe_status s);
/* Library version string. */
const char* moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
