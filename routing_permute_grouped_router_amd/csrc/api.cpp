// C ABI of the MoE hot path: argument validation and kernel launches.
// Every entry point only enqueues work on the caller's stream (no allocation,
// no synchronisation, no device-to-host copy).
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "moe_internal.h"

using namespace moe;

namespace {

thread_local char g_err[512] = "";

moe_status fail(moe_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

moe_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return MOE_OK;
    if (e == hipErrorNotSupported) return fail(MOE_ERR_UNSUPPORTED, "%s: not built for this configuration", what);
    return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Every device array is read and written in 16-byte vectors.
#define ALIGNED16(ptr)                                                                                  \
    do {                                                                                                \
        if ((uintptr_t)(ptr) % 16) return fail(MOE_ERR_INVALID_ARG, "%s is not 16-byte aligned", #ptr); \
    } while (0)
#define REQUIRE(ptr)                                                              \
    do {                                                                          \
        if ((ptr) == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s is NULL", #ptr); \
        ALIGNED16(ptr);                                                           \
    } while (0)

int64_t rows_capacity(const moe_config& c) { return (int64_t)c.T * c.k + (int64_t)c.E * (c.align - 1); }
bool is_mx(const moe_config& c) { return c.dtype == MOE_MXFP8 || c.dtype == MOE_MXFP4; }

// Sizes and enums; does not look at pointers.
moe_status check_config(const moe_config* cfg) {
    if (!cfg) return fail(MOE_ERR_INVALID_ARG, "cfg is NULL");
    const moe_config& c = *cfg;
    if (c.T < 0) return fail(MOE_ERR_INVALID_ARG, "T must be >= 0 (got %d)", c.T);
    if (c.E < 1 || c.E > kMaxExperts) return fail(MOE_ERR_INVALID_ARG, "E must be in [1, %d] (got %d)", kMaxExperts, c.E);
    if (c.k < 1 || c.k > c.E || c.k > kMaxTopK)
        return fail(MOE_ERR_INVALID_ARG, "k must be in [1, min(E, %d)] (got k=%d, E=%d)", kMaxTopK, c.k, c.E);
    if (c.align < 1) return fail(MOE_ERR_INVALID_ARG, "align must be >= 1 (got %d)", c.align);
    if (c.H < 1 || c.F < 1) return fail(MOE_ERR_INVALID_ARG, "H and F must be positive (got H=%d, F=%d)", c.H, c.F);
    if (c.score != MOE_SOFTMAX && c.score != MOE_SIGMOID)
        return fail(MOE_ERR_INVALID_ARG, "score must be MOE_SOFTMAX or MOE_SIGMOID (got %d)", c.score);
    if (c.renorm != 0 && c.renorm != 1) return fail(MOE_ERR_INVALID_ARG, "renorm must be 0 or 1 (got %d)", c.renorm);
    if (c.dtype != MOE_F32 && c.dtype != MOE_BF16 && c.dtype != MOE_MXFP8 && c.dtype != MOE_MXFP4)
        return fail(MOE_ERR_INVALID_ARG, "dtype must be MOE_F32, MOE_BF16, MOE_MXFP8 or MOE_MXFP4 (got %d)", c.dtype);
    if (c.weight_site != MOE_WEIGHT_AT_COMBINE && c.weight_site != MOE_WEIGHT_AT_FC1 &&
        c.weight_site != MOE_WEIGHT_AT_FC2)
        return fail(MOE_ERR_INVALID_ARG, "weight_site must be MOE_WEIGHT_AT_COMBINE, _FC1 or _FC2 (got %d)",
                    c.weight_site);
    if (!(c.swiglu_limit >= 0.f) || c.swiglu_limit == INFINITY)
        return fail(MOE_ERR_INVALID_ARG, "swiglu_limit must be finite and >= 0 (got %g)", (double)c.swiglu_limit);
    if (rows_capacity(c) >= (int64_t)1 << 31)
        return fail(MOE_ERR_INVALID_ARG, "T*k + E*(align-1) must be below 2^31");
    if ((int64_t)c.T * c.H >= (int64_t)1 << 40) return fail(MOE_ERR_INVALID_ARG, "T*H too large");
    return MOE_OK;
}

// Shapes the GEMM and row kernels are built for.
moe_status check_shapes(const moe_config& c) {
    if (c.H % 128 != 0) return fail(MOE_ERR_UNSUPPORTED, "H must be a multiple of 128 (got %d)", c.H);
    if (c.F % 64 != 0) return fail(MOE_ERR_UNSUPPORTED, "F must be a multiple of 64 (got %d)", c.F);
    // one expert's weights are addressed with 32-bit byte offsets
    if ((int64_t)c.F * c.H >= (int64_t)1 << 29)
        return fail(MOE_ERR_UNSUPPORTED, "F*H must be below 2^29 (got F=%d, H=%d)", c.F, c.H);
    if (c.dtype == MOE_MXFP8 && c.F % 128 != 0)
        return fail(MOE_ERR_UNSUPPORTED, "MXFP8 needs F to be a multiple of 128 (got %d)", c.F);
    // MXFP4: a 128-byte GEMM stage holds 256 values, and one 16-byte load
    // brings a row's scales of two stages
    if (c.dtype == MOE_MXFP4 && (c.H % 512 != 0 || c.F % 512 != 0))
        return fail(MOE_ERR_UNSUPPORTED, "MXFP4 needs H and F to be multiples of 512 (got H=%d, F=%d)", c.H, c.F);
    return MOE_OK;
}

moe_status check_ws(const moe_config& c, const void* ws, size_t ws_bytes, bool backward = false) {
    const size_t need = backward ? moe_backward_workspace_size(&c) : moe_workspace_size(&c);
    if (need == 0) return MOE_OK;
    if (ws == nullptr || ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes required (got %zu%s)", need, ws_bytes,
                    ws ? "" : ", ws is NULL");
    return MOE_OK;
}

hipStream_t as_stream(void* s) { return (hipStream_t)s; }

size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

// Forward workspace: the grouping's per-chunk counts, then the GEMMs' region
// (work-queue counters and split-tile partial sums; used in stream order by
// the gate/up GEMM and then the down GEMM).
size_t group_ws_bytes(const moe_config& c) { return round256((size_t)group_n_chunks(c.T, c.E) * c.E * sizeof(int32_t)); }
void* gemm_ws(const moe_config& c, void* ws) { return (char*)ws + group_ws_bytes(c); }

// Per-row copy of the routing weights (epilogue placements), after the
// forward region of the workspace.
size_t row_w_ws_bytes(const moe_config& c) { return round256((size_t)(rows_capacity(c) + kRowWeightPad) * sizeof(float)); }
float* row_w_ws(const moe_config& c, void* ws) {
    return (float*)((char*)ws + group_ws_bytes(c) + round256(gemm_bf16_ws_bytes(c) + gemm_mxfp8_ws_bytes(c)));
}

// The gate/up GEMM with all its forms: gsrc/gcounts non-null = gather form
// (a is x), row_w non-null = h scaled by the row's routing weight.
moe_status swiglu_checked(const moe_config* cfg, const void* a, const uint8_t* a_scale, const void* w1,
                          const uint8_t* w1_scale, const int32_t* offsets, void* h, uint8_t* h_scale, void* stash,
                          const int32_t* gsrc, const int32_t* gcounts, const float* row_w, void* ws, size_t ws_bytes,
                          void* stream, const char* what, bool launch = true) {
    moe_status st = check_config(cfg);
    if (st) return st;
    const moe_config& c = *cfg;
    if ((st = check_shapes(c))) return st;
    if (rows_capacity(c) == 0) return MOE_OK;
    // the gather form addresses a row of x with a 32-bit byte offset
    if (gsrc && (int64_t)c.T * c.H * (c.dtype == MOE_F32 ? 8 : c.dtype == MOE_BF16 ? 4 : c.dtype == MOE_MXFP8 ? 2 : 1) >=
                    ((int64_t)1 << 33))
        return fail(MOE_ERR_UNSUPPORTED, "%s: the gather form needs T*H*element size < 4 GiB", what);
    if (!a) return fail(MOE_ERR_INVALID_ARG, "%s: the grouped operand (xp or x) is NULL", what);
    REQUIRE(w1);
    REQUIRE(offsets);
    REQUIRE(h);
    if ((st = check_ws(c, ws, ws_bytes))) return st;
    if (is_mx(c)) {
        if (!a_scale) return fail(MOE_ERR_INVALID_ARG, "%s: the grouped operand's MX scales are NULL", what);
        REQUIRE(w1_scale);
        REQUIRE(h_scale);
    }
    if (!launch) return MOE_OK;  // arguments checked, nothing enqueued
    hipStream_t s = as_stream(stream);
    switch (c.dtype) {
    case MOE_BF16:
        return hip_status(launch_swiglu_gemm_bf16(c, (const uint16_t*)a, (const uint16_t*)w1, offsets, (uint16_t*)h,
                                                  (uint16_t*)stash, gsrc, gcounts, row_w, gemm_ws(c, ws), s),
                          what);
    case MOE_F32:
        return hip_status(launch_swiglu_gemm_f32(c, (const float*)a, (const float*)w1, offsets, (float*)h,
                                                 (float*)stash, gsrc, gcounts, row_w, s),
                          what);
    default:  // MXFP8 and MXFP4
        return hip_status(launch_swiglu_gemm_mxfp8(c, (const uint8_t*)a, a_scale, (const uint8_t*)w1, w1_scale,
                                                   offsets, (uint8_t*)h, h_scale, (uint16_t*)stash, gsrc, gcounts,
                                                   row_w, gemm_ws(c, ws), s),
                          what);
    }
}

// The down GEMM; row_w non-null = Yp scaled by the row's routing weight.
moe_status down_checked(const moe_config* cfg, const void* h, const uint8_t* h_scale, const void* w2,
                        const uint8_t* w2_scale, const int32_t* offsets, void* yp, const float* row_w, void* ws,
                        size_t ws_bytes, void* stream, const char* what, bool launch = true) {
    moe_status st = check_config(cfg);
    if (st) return st;
    const moe_config& c = *cfg;
    if ((st = check_shapes(c))) return st;
    if (rows_capacity(c) == 0) return MOE_OK;
    REQUIRE(h);
    REQUIRE(w2);
    REQUIRE(offsets);
    REQUIRE(yp);
    if ((st = check_ws(c, ws, ws_bytes))) return st;
    if (is_mx(c)) {
        REQUIRE(h_scale);
        REQUIRE(w2_scale);
    }
    if (!launch) return MOE_OK;  // arguments checked, nothing enqueued
    hipStream_t s = as_stream(stream);
    switch (c.dtype) {
    case MOE_BF16:
        return hip_status(launch_down_gemm_bf16(c, (const uint16_t*)h, (const uint16_t*)w2, offsets, (uint16_t*)yp,
                                                row_w, gemm_ws(c, ws), s),
                          what);
    case MOE_F32:
        return hip_status(launch_down_gemm_f32(c, (const float*)h, (const float*)w2, offsets, (float*)yp, row_w, s),
                          what);
    default:  // MXFP8 and MXFP4
        return hip_status(launch_down_gemm_mxfp8(c, (const uint8_t*)h, h_scale, (const uint8_t*)w2, w2_scale, offsets,
                                                 (uint16_t*)yp, row_w, gemm_ws(c, ws), s),
                          what);
    }
}

// Writes the per-row routing weights into the workspace; *row_w = their
// address (left null when there are no rows).
moe_status row_weights_checked(const moe_config* cfg, const int32_t* src_map, const float* w, void* ws,
                               size_t ws_bytes, void* stream, const float** row_w, bool launch = true) {
    moe_status st = check_config(cfg);
    if (st) return st;
    const moe_config& c = *cfg;
    if (rows_capacity(c) == 0) return MOE_OK;
    REQUIRE(src_map);
    REQUIRE(w);
    if ((st = check_ws(c, ws, ws_bytes))) return st;
    if (!launch) return MOE_OK;
    float* rw = row_w_ws(c, ws);
    if ((st = hip_status(launch_row_weights(c, src_map, w, rw, as_stream(stream)), "row weights"))) return st;
    *row_w = rw;
    return MOE_OK;
}

moe_status route_checked(const moe_config* cfg, const float* logits, const float* bias, int32_t* idx, float* w,
                         void* stream, bool launch) {
    moe_status st = check_config(cfg);
    if (st) return st;
    if (cfg->T > 0) {
        REQUIRE(logits);
        REQUIRE(idx);
        REQUIRE(w);
        ALIGNED16(bias);  // optional
    }
    if (!launch) return MOE_OK;
    return hip_status(launch_route(*cfg, logits, bias, idx, w, as_stream(stream)), "moe_route");
}

moe_status permute_checked(const moe_config* cfg, const void* x, const uint8_t* x_scale, const int32_t* idx,
                           void* xp, uint8_t* xp_scale, int32_t* counts, int32_t* offsets, int32_t* row_map,
                           int32_t* src_map, int32_t* err, void* ws, size_t ws_bytes, void* stream, bool launch) {
    moe_status st = check_config(cfg);
    if (st) return st;
    const moe_config& c = *cfg;
    if (is_mx(c) && c.H % 128) return fail(MOE_ERR_UNSUPPORTED, "the MX formats need H %% 128 == 0");
    REQUIRE(counts);
    REQUIRE(offsets);
    if (rows_capacity(c) > 0) REQUIRE(src_map);
    if (c.T > 0) {
        REQUIRE(idx);
        REQUIRE(row_map);
        if (xp) {  // xp NULL: the grouping only (for the gather form of the gate/up GEMM)
            REQUIRE(x);
            if (is_mx(c)) {
                REQUIRE(x_scale);
                REQUIRE(xp_scale);
            }
        }
    }
    if ((st = check_ws(c, ws, ws_bytes))) return st;
    if (!launch) return MOE_OK;
    return hip_status(launch_group(c, idx, x, x_scale, xp, xp_scale, counts, offsets, row_map, src_map, err,
                                   (int32_t*)ws, as_stream(stream)),
                      "moe_permute");
}

moe_status combine_checked(const moe_config* cfg, const void* yp, const int32_t* row_map, const float* w, void* y,
                           void* stream, bool launch) {
    moe_status st = check_config(cfg);
    if (st) return st;
    if ((st = check_shapes(*cfg))) return st;
    if (cfg->T > 0) {
        REQUIRE(yp);
        REQUIRE(row_map);
        REQUIRE(y);
    }
    if (!launch) return MOE_OK;
    return hip_status(launch_combine(*cfg, yp, row_map, w, y, as_stream(stream)), "moe_combine");
}

// The backward is built for bf16 storage with the routing weights applied in
// the combine.
moe_status check_backward(const moe_config* cfg) {
    moe_status st = check_config(cfg);
    if (st) return st;
    if (cfg->dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "the backward is built for BF16 storage");
    if (cfg->weight_site != MOE_WEIGHT_AT_COMBINE)
        return fail(MOE_ERR_UNSUPPORTED, "the backward is built for the weights applied in the combine");
    return check_shapes(*cfg);
}

moe_status combine_bwd_checked(const moe_config* cfg, const void* dy, const int32_t* row_map, const int32_t* src_map,
                               const int32_t* offsets, const float* w, void* dyp, void* stream, bool launch) {
    moe_status st = check_backward(cfg);
    if (st) return st;
    REQUIRE(offsets);
    if (rows_capacity(*cfg) > 0) {
        REQUIRE(dy);
        REQUIRE(row_map);
        REQUIRE(src_map);
        REQUIRE(w);
        REQUIRE(dyp);
    }
    if (!launch) return MOE_OK;
    return hip_status(launch_combine_bwd(*cfg, dy, row_map, src_map, offsets, w, dyp, as_stream(stream)),
                      "moe_combine_bwd");
}

moe_status down_bwd_checked(const moe_config* cfg, const void* dyp, const void* w2, const void* h,
                            const void* gu_stash, const int32_t* offsets, void* dgu, float* dw2, void* ws,
                            size_t ws_bytes, void* stream, bool launch) {
    moe_status st = check_backward(cfg);
    if (st) return st;
    REQUIRE(w2);
    REQUIRE(dw2);
    REQUIRE(offsets);
    if ((st = check_ws(*cfg, ws, ws_bytes, true))) return st;
    if (rows_capacity(*cfg) > 0) {
        REQUIRE(dyp);
        REQUIRE(h);
        REQUIRE(gu_stash);
        REQUIRE(dgu);
    }
    if (!launch) return MOE_OK;
    return hip_status(launch_down_bwd(*cfg, dyp, w2, h, gu_stash, offsets, dgu, dw2, ws, as_stream(stream)),
                      "moe_grouped_down_bwd");
}

moe_status swiglu_bwd_checked(const moe_config* cfg, const void* dgu, const void* w1, const void* xp,
                              const int32_t* offsets, void* dxp, float* dw1, void* ws, size_t ws_bytes, void* stream,
                              bool launch) {
    moe_status st = check_backward(cfg);
    if (st) return st;
    REQUIRE(w1);
    REQUIRE(dw1);
    REQUIRE(offsets);
    if ((st = check_ws(*cfg, ws, ws_bytes, true))) return st;
    if (rows_capacity(*cfg) > 0) {
        REQUIRE(dgu);
        REQUIRE(xp);
        REQUIRE(dxp);
    }
    if (!launch) return MOE_OK;
    return hip_status(launch_swiglu_bwd(*cfg, dgu, w1, xp, offsets, dxp, dw1, ws, as_stream(stream)),
                      "moe_grouped_swiglu_bwd");
}

moe_status permute_bwd_checked(const moe_config* cfg, const void* dxp, const int32_t* row_map, void* dx,
                               void* stream, bool launch) {
    moe_status st = check_backward(cfg);
    if (st) return st;
    if (cfg->T > 0) {
        REQUIRE(dxp);
        REQUIRE(row_map);
        REQUIRE(dx);
    }
    if (!launch) return MOE_OK;
    return hip_status(launch_permute_bwd(*cfg, dxp, row_map, dx, as_stream(stream)), "moe_permute_bwd");
}

}  // namespace

moe_status moe::set_error(moe_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

extern "C" {

int64_t moe_rows_capacity(const moe_config* cfg) {
    if (check_config(cfg) != MOE_OK) return -1;
    return rows_capacity(*cfg);
}

size_t moe_workspace_size(const moe_config* cfg) {
    if (check_config(cfg) != MOE_OK) return 0;
    const moe_config& c = *cfg;
    return group_ws_bytes(c) + round256(gemm_bf16_ws_bytes(c) + gemm_mxfp8_ws_bytes(c)) + row_w_ws_bytes(c);
}

size_t moe_backward_workspace_size(const moe_config* cfg) {
    if (check_config(cfg) != MOE_OK) return 0;
    return cfg->dtype == MOE_BF16 ? round256(bwd_workspace_bytes(*cfg)) : 0;
}

moe_status moe_route(const moe_config* cfg, const float* logits, const float* bias, int32_t* idx, float* w,
                     void* stream) {
    return route_checked(cfg, logits, bias, idx, w, stream, true);
}

moe_status moe_permute(const moe_config* cfg, const void* x, const uint8_t* x_scale, const int32_t* idx, void* xp,
                       uint8_t* xp_scale, int32_t* counts, int32_t* offsets, int32_t* row_map, int32_t* src_map,
                       int32_t* err, void* ws, size_t ws_bytes, void* stream) {
    // checked in full before the grouping is launched
    moe_status st = permute_checked(cfg, x, x_scale, idx, xp, xp_scale, counts, offsets, row_map, src_map, err, ws,
                                    ws_bytes, stream, false);
    if (st) return st;
    return permute_checked(cfg, x, x_scale, idx, xp, xp_scale, counts, offsets, row_map, src_map, err, ws, ws_bytes,
                           stream, true);
}

moe_status moe_grouped_swiglu_gemm(const moe_config* cfg, const void* xp, const uint8_t* xp_scale, const void* w1,
                                   const uint8_t* w1_scale, const int32_t* offsets, void* h, uint8_t* h_scale,
                                   void* gu_stash, void* ws, size_t ws_bytes, void* stream) {
    return swiglu_checked(cfg, xp, xp_scale, w1, w1_scale, offsets, h, h_scale, gu_stash, nullptr, nullptr, nullptr,
                          ws, ws_bytes, stream, "moe_grouped_swiglu_gemm");
}

moe_status moe_grouped_swiglu_gemm_gather(const moe_config* cfg, const void* x, const uint8_t* x_scale,
                                          const int32_t* src_map, const int32_t* counts, const void* w1,
                                          const uint8_t* w1_scale, const int32_t* offsets, void* h, uint8_t* h_scale,
                                          void* ws, size_t ws_bytes, void* stream) {
    if (cfg && rows_capacity(*cfg) > 0) {
        REQUIRE(src_map);
        REQUIRE(counts);
    }
    return swiglu_checked(cfg, x, x_scale, w1, w1_scale, offsets, h, h_scale, nullptr, src_map, counts, nullptr, ws,
                          ws_bytes, stream, "moe_grouped_swiglu_gemm_gather");
}

moe_status moe_grouped_swiglu_gemm_weighted(const moe_config* cfg, const void* xp, const uint8_t* xp_scale,
                                            const void* w1, const uint8_t* w1_scale, const int32_t* offsets,
                                            const int32_t* src_map, const float* w, void* h, uint8_t* h_scale,
                                            void* ws, size_t ws_bytes, void* stream) {
    // every argument is checked before the per-row weights are launched
    moe_status st = swiglu_checked(cfg, xp, xp_scale, w1, w1_scale, offsets, h, h_scale, nullptr, nullptr, nullptr,
                                   nullptr, ws, ws_bytes, stream, "moe_grouped_swiglu_gemm_weighted", false);
    if (st) return st;
    const float* row_w = nullptr;
    if ((st = row_weights_checked(cfg, src_map, w, ws, ws_bytes, stream, &row_w))) return st;
    return swiglu_checked(cfg, xp, xp_scale, w1, w1_scale, offsets, h, h_scale, nullptr, nullptr, nullptr, row_w, ws,
                          ws_bytes, stream, "moe_grouped_swiglu_gemm_weighted");
}

moe_status moe_grouped_down_gemm(const moe_config* cfg, const void* h, const uint8_t* h_scale, const void* w2,
                                 const uint8_t* w2_scale, const int32_t* offsets, void* yp, void* ws, size_t ws_bytes,
                                 void* stream) {
    return down_checked(cfg, h, h_scale, w2, w2_scale, offsets, yp, nullptr, ws, ws_bytes, stream,
                        "moe_grouped_down_gemm");
}

moe_status moe_grouped_down_gemm_weighted(const moe_config* cfg, const void* h, const uint8_t* h_scale,
                                          const void* w2, const uint8_t* w2_scale, const int32_t* offsets,
                                          const int32_t* src_map, const float* w, void* yp, void* ws,
                                          size_t ws_bytes, void* stream) {
    // every argument is checked before the per-row weights are launched
    moe_status st = down_checked(cfg, h, h_scale, w2, w2_scale, offsets, yp, nullptr, ws, ws_bytes, stream,
                                 "moe_grouped_down_gemm_weighted", false);
    if (st) return st;
    const float* row_w = nullptr;
    if ((st = row_weights_checked(cfg, src_map, w, ws, ws_bytes, stream, &row_w))) return st;
    return down_checked(cfg, h, h_scale, w2, w2_scale, offsets, yp, row_w, ws, ws_bytes, stream,
                        "moe_grouped_down_gemm_weighted");
}

moe_status moe_combine(const moe_config* cfg, const void* yp, const int32_t* row_map, const float* w, void* y,
                       void* stream) {
    return combine_checked(cfg, yp, row_map, w, y, stream, true);
}

// Both fused calls check every step's arguments (pass 0) before the first
// launch (pass 1), so a host-checkable problem enqueues nothing.
moe_status moe_forward(const moe_config* cfg, const float* logits, const float* bias, const void* x,
                       const uint8_t* x_scale, const void* w1, const uint8_t* w1_scale, const void* w2,
                       const uint8_t* w2_scale, void* y,
                       int32_t* idx, float* w, int32_t* counts, int32_t* offsets, int32_t* row_map,
                       int32_t* src_map, void* xp, uint8_t* xp_scale, void* h, uint8_t* h_scale, void* yp,
                       void* gu_stash, int32_t* err, void* ws, size_t ws_bytes, void* stream) {
    moe_status st = check_config(cfg);
    if (st) return st;
    const moe_config& c = *cfg;
    if ((st = check_shapes(c))) return st;
    REQUIRE(w1);
    REQUIRE(w2);
    if (is_mx(c)) {
        REQUIRE(w1_scale);
        REQUIRE(w2_scale);
    }
    if (!xp && gu_stash) return fail(MOE_ERR_INVALID_ARG, "a training forward (gu_stash) needs xp");
    if (!xp && rows_capacity(c) > 0) REQUIRE(src_map);
    const bool at_combine = c.weight_site == MOE_WEIGHT_AT_COMBINE;
    for (int pass = 0; pass < 2; ++pass) {
        const bool launch = pass == 1;
        if ((st = route_checked(cfg, logits, bias, idx, w, stream, launch))) return st;
        if ((st = permute_checked(cfg, x, x_scale, idx, xp, xp_scale, counts, offsets, row_map, src_map, err, ws,
                                  ws_bytes, stream, launch)))
            return st;
        // the routing weights applied in an expert epilogue: their per-row copy
        const float* row_w = nullptr;
        if (!at_combine && (st = row_weights_checked(cfg, src_map, w, ws, ws_bytes, stream, &row_w, launch)))
            return st;
        const float* fc1_w = c.weight_site == MOE_WEIGHT_AT_FC1 ? row_w : nullptr;
        const float* fc2_w = c.weight_site == MOE_WEIGHT_AT_FC2 ? row_w : nullptr;
        if (xp)
            st = swiglu_checked(cfg, xp, xp_scale, w1, w1_scale, offsets, h, h_scale, gu_stash, nullptr, nullptr,
                                fc1_w, ws, ws_bytes, stream, "moe_forward", launch);
        else
            st = swiglu_checked(cfg, x, x_scale, w1, w1_scale, offsets, h, h_scale, nullptr, src_map, counts, fc1_w,
                                ws, ws_bytes, stream, "moe_forward", launch);
        if (st) return st;
        if ((st = down_checked(cfg, h, h_scale, w2, w2_scale, offsets, yp, fc2_w, ws, ws_bytes, stream, "moe_forward",
                               launch)))
            return st;
        if ((st = combine_checked(cfg, yp, row_map, at_combine ? w : nullptr, y, stream, launch))) return st;
    }
    return MOE_OK;
}

moe_status moe_route_bwd(const moe_config* cfg, const void* dy, const void* yp, const float* logits,
                         const int32_t* idx, const int32_t* row_map, float* dw, float* dlogits, void* stream) {
    moe_status st = check_config(cfg);
    if (st) return st;
    if ((st = check_shapes(*cfg))) return st;
    if (cfg->weight_site != MOE_WEIGHT_AT_COMBINE)
        return fail(MOE_ERR_UNSUPPORTED, "the routing backward reads unweighted Yp rows (weights applied in the combine)");
    if (cfg->T == 0) return MOE_OK;
    REQUIRE(dy);
    REQUIRE(yp);
    REQUIRE(logits);
    REQUIRE(idx);
    REQUIRE(row_map);
    REQUIRE(dlogits);
    return hip_status(launch_route_bwd(*cfg, dy, yp, logits, idx, row_map, dw, dlogits, as_stream(stream)),
                      "moe_route_bwd");
}

moe_status moe_combine_bwd(const moe_config* cfg, const void* dy, const int32_t* row_map, const int32_t* src_map,
                           const int32_t* offsets, const float* w, void* dyp, void* stream) {
    return combine_bwd_checked(cfg, dy, row_map, src_map, offsets, w, dyp, stream, true);
}

moe_status moe_grouped_down_bwd(const moe_config* cfg, const void* dyp, const void* w2, const void* h,
                                const void* gu_stash, const int32_t* offsets, void* dgu, float* dw2, void* ws,
                                size_t ws_bytes, void* stream) {
    return down_bwd_checked(cfg, dyp, w2, h, gu_stash, offsets, dgu, dw2, ws, ws_bytes, stream, true);
}

moe_status moe_grouped_swiglu_bwd(const moe_config* cfg, const void* dgu, const void* w1, const void* xp,
                                  const int32_t* offsets, void* dxp, float* dw1, void* ws, size_t ws_bytes,
                                  void* stream) {
    return swiglu_bwd_checked(cfg, dgu, w1, xp, offsets, dxp, dw1, ws, ws_bytes, stream, true);
}

moe_status moe_permute_bwd(const moe_config* cfg, const void* dxp, const int32_t* row_map, void* dx, void* stream) {
    return permute_bwd_checked(cfg, dxp, row_map, dx, stream, true);
}

moe_status moe_backward(const moe_config* cfg, const void* dy, const float* w, const void* w1, const void* w2,
                        const int32_t* offsets, const int32_t* row_map, const int32_t* src_map, const void* xp,
                        const void* h, const void* gu_stash, void* dyp, void* dgu, void* dxp, void* dx, float* dw1,
                        float* dw2, void* ws, size_t ws_bytes, void* stream) {
    moe_status st;
    for (int pass = 0; pass < 2; ++pass) {
        const bool launch = pass == 1;
        if ((st = combine_bwd_checked(cfg, dy, row_map, src_map, offsets, w, dyp, stream, launch))) return st;
        if ((st = down_bwd_checked(cfg, dyp, w2, h, gu_stash, offsets, dgu, dw2, ws, ws_bytes, stream, launch)))
            return st;
        if ((st = swiglu_bwd_checked(cfg, dgu, w1, xp, offsets, dxp, dw1, ws, ws_bytes, stream, launch))) return st;
        if ((st = permute_bwd_checked(cfg, dxp, row_map, dx, stream, launch))) return st;
    }
    return MOE_OK;
}

moe_status moe_quantize_mxfp8(const float* in, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                              void* stream) {
    if (rows < 0 || cols < 0) return fail(MOE_ERR_INVALID_ARG, "rows and cols must be >= 0");
    if (cols % kMxBlock) return fail(MOE_ERR_INVALID_ARG, "cols must be a multiple of 32 (got %lld)", (long long)cols);
    if (rows * cols > 0) {
        REQUIRE(in);
        REQUIRE(codes);
        REQUIRE(scales);
    }
    return hip_status(launch_quantize_mxfp8(in, rows, cols, codes, scales, as_stream(stream)), "moe_quantize_mxfp8");
}

moe_status moe_quantize_mxfp4(const float* in, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                              void* stream) {
    if (rows < 0 || cols < 0) return fail(MOE_ERR_INVALID_ARG, "rows and cols must be >= 0");
    if (cols % kMxBlock) return fail(MOE_ERR_INVALID_ARG, "cols must be a multiple of 32 (got %lld)", (long long)cols);
    if (rows * cols > 0) {
        REQUIRE(in);
        REQUIRE(codes);
        REQUIRE(scales);
    }
    return hip_status(launch_quantize_mxfp4(in, rows, cols, codes, scales, as_stream(stream)), "moe_quantize_mxfp4");
}

const char* moe_last_error(void) { return g_err; }

const char* moe_status_string(moe_status s) {
    switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    }
    return "MOE_ERR_UNKNOWN";
}

const char* moe_version(void) { return "moe-gfx950 0.1"; }

}  // extern "C"
