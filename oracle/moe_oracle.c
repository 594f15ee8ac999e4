/*
 * moe_oracle.c -- plain, slow CPU oracle for the single-GPU MoE FFN hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file: only tests/, the smoke check and the CPU-baseline leg of the
 * benchmark do.  It shares no code, header, table or constant with the HIP
 * library under routing_permute_grouped_router_amd/csrc.
 *
 * Sources (web pages; cited by title and section):
 *   [TE-EP]   "[JAX] Expert Parallelism: JAX primitives + VJPs"
 *             (TransformerEngine PR #3036), Summary and the squashed commit
 *             messages quoted on that page.
 *   [CUDNN]   "Add MoE + expert-parallel Python API surface, PyTorch reference,
 *             and tests" (cudnn-frontend PR #389), Summary and the review
 *             comments quoting MoeEp.__call__ / backward / BlockScaledTensor.
 *   [ISSUE]   "MoE training optimization" (TransformerEngine issue #2438).
 *   [BLOCK]   "[Draft][JAX] MoE block optimization" (TransformerEngine
 *             PR #3638), Diagram.
 *   [OCP-MX]  OCP Microscaling Formats (MX) Specification v1.0 (public), for
 *             the MXFP8 E4M3 element format and the E8M0 shared scale.
 *
 * Arithmetic: every stored value is decoded exactly to double; every sum is
 * accumulated in double in a fixed ascending order; results are rounded once to
 * the storage format at the points the method stores them (h, Yp, y, the
 * backward tensors).  Transcendentals use libm in double.
 *
 * Parity pins: every function below is checked by tests/test_oracle_*.py
 * against closed forms, invariants, library routines (numpy/torch/scipy) and
 * brute force on tiny inputs.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Storage formats understood by the oracle (its own numbering). */
enum { OR_F32 = 0, OR_BF16 = 1, OR_MXFP8 = 2, OR_MXFP4 = 3 };
/* Score functions. */
enum { OR_SOFTMAX = 0, OR_SIGMOID = 1 };

#define OR_MX_BLOCK 32

/*
 * Optional SwiGLU clamp ([CUDNN] Summary: local SwiGLU experts with an
 * optional DeepSeek-style clamp; the pages state no bounds).  With a limit
 * L > 0 the gate is clamped from above and the up projection to [-L, L]
 * before the activation:
 *   h = silu(min(g, L)) * clamp(u, -L, L)
 * and the gradient of each clamp passes where its bound is not exceeded (the
 * bounds themselves included).  L = 0: no clamp.  The limit is set per call
 * by the Python wrapper (or_set_swiglu_limit) before the function using it.
 */
static double or_limit = 0.0;
void or_set_swiglu_limit(double limit) { or_limit = limit; }

static double or_swiglu(double g, double u) {
    if (or_limit > 0.0) {
        g = g > or_limit ? or_limit : g;
        u = u > or_limit ? or_limit : (u < -or_limit ? -or_limit : u);
    }
    return (g / (1.0 + exp(-g))) * u;
}

/* Partial derivatives dh/dg and dh/du of or_swiglu at the unclamped (g, u). */
static void or_swiglu_grad(double g, double u, double* dg, double* du) {
    double mg = 1.0, mu = 1.0;
    if (or_limit > 0.0) {
        if (g > or_limit) { g = or_limit; mg = 0.0; }
        if (u > or_limit) { u = or_limit; mu = 0.0; }
        if (u < -or_limit) { u = -or_limit; mu = 0.0; }
    }
    const double sig = 1.0 / (1.0 + exp(-g));
    *dg = mg * u * sig * (1.0 + g * (1.0 - sig));
    *du = mu * g * sig;
}

/* Where the routing weight is applied (its own numbering). */
enum { OR_AT_COMBINE = 0, OR_AT_FC1 = 1, OR_AT_FC2 = 2 };

/* ------------------------------------------------------------------------ */
/* Number formats                                                           */
/* ------------------------------------------------------------------------ */

/* bfloat16: the upper 16 bits of an IEEE binary32.  Conversion from a double
 * is a single round-to-nearest-even straight to the 8-bit significand (no
 * detour through binary32, which could round twice). */
uint16_t or_bf16_from_double(double v) {
    if (isnan(v)) return (uint16_t)(signbit(v) ? 0xFFC0u : 0x7FC0u);
    if (v == 0.0) return (uint16_t)(signbit(v) ? 0x8000u : 0x0000u);
    const int neg = v < 0.0;
    double a = fabs(v);
    /* bf16 normal range: 2^-126 .. (2 - 2^-7) * 2^127; subnormals have a
     * quantum of 2^-133. */
    int e2;
    frexp(a, &e2);          /* a = m * 2^e2, m in [0.5, 1) */
    int e = e2 - 1;         /* a in [2^e, 2^(e+1)) */
    if (e < -126) e = -126; /* subnormal range keeps the 2^-133 quantum */
    double quantum = ldexp(1.0, e - 7);
    double q = nearbyint(a / quantum); /* exact division (power of two); RNE */
    double r = q * quantum;
    uint16_t bits;
    if (r >= ldexp(1.0, 128)) {
        bits = 0x7F80u; /* overflow to infinity */
    } else {
        /* Encode r exactly: it is a bf16 value. */
        float f = (float)r; /* exact: r has <= 8 significant bits */
        uint32_t u;
        memcpy(&u, &f, 4);
        bits = (uint16_t)(u >> 16);
    }
    return (uint16_t)(bits | (neg ? 0x8000u : 0u));
}

double or_double_from_bf16(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* OCP E4M3 ("E4M3FN"): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits,
 * no infinities, S.1111.111 is NaN, largest finite 448, smallest subnormal
 * 2^-9 [OCP-MX, element formats]. */
double or_double_from_e4m3(uint8_t c) {
    const int s = c >> 7, ex = (c >> 3) & 0xF, m = c & 7;
    double v;
    if (ex == 0xF && m == 7) return NAN;
    if (ex == 0) v = ldexp((double)m, -9);            /* m/8 * 2^-6 */
    else v = ldexp(8.0 + (double)m, ex - 7 - 3);        /* (1+m/8) * 2^(ex-7) */
    return s ? -v : v;
}

/* Round-to-nearest-even to E4M3, saturating to +-448 (the MX conversion
 * clamps values beyond the element format's largest normal). */
uint8_t or_e4m3_from_double(double v) {
    if (isnan(v)) return 0x7F;
    const uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs(v);
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);
    int e = e2 - 1;          /* a in [2^e, 2^(e+1)) */
    if (e < -6) e = -6;      /* subnormal quantum 2^-9 */
    double quantum = ldexp(1.0, e - 3);
    double q = nearbyint(a / quantum);
    double r = q * quantum;
    if (r > 448.0) r = 448.0;
    /* encode r (an E4M3 value) */
    if (r < ldexp(1.0, -6)) {
        int m = (int)(r / ldexp(1.0, -9));
        return (uint8_t)(sign | m);
    }
    frexp(r, &e2);
    e = e2 - 1;
    int m = (int)(r / ldexp(1.0, e - 3)) - 8;
    return (uint8_t)(sign | ((e + 7) << 3) | m);
}

/* OCP E2M1 ("FP4"): 1 sign, 2 exponent bits (bias 1), 1 mantissa bit, no
 * infinities or NaN [OCP-MX, element formats]: magnitudes 0 and 0.5
 * (subnormal), 1, 1.5, 2, 3, 4, 6.  A code is the low 4 bits of c. */
double or_double_from_e2m1(uint8_t c) {
    const int s = (c >> 3) & 1, ex = (c >> 1) & 3, m = c & 1;
    const double v = ex == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, ex - 1);
    return s ? -v : v;
}

/* Round-to-nearest-even to E2M1, saturating to +-6 (the MX conversion clamps
 * values beyond the element format's largest normal).  The quantum is
 * 2^(e-1) for |v| in [2^e, 2^(e+1)), e >= 0, and the subnormal 0.5 below 1;
 * nearbyint's ties to even land on the even mantissa. */
uint8_t or_e2m1_from_double(double v) {
    const uint8_t sign = signbit(v) ? 0x8 : 0x0;
    if (isnan(v)) return (uint8_t)(sign | 0x7);
    const double a = fabs(v);
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);
    int e = e2 - 1; /* a in [2^e, 2^(e+1)) */
    if (e < 0) e = 0;
    const double quantum = ldexp(1.0, e - 1);
    double r = nearbyint(a / quantum) * quantum;
    if (r > 6.0) r = 6.0;
    if (r < 1.0) return (uint8_t)(sign | (int)(r / 0.5)); /* 0 or 0.5 */
    frexp(r, &e2);
    e = e2 - 1;
    const int m = (int)(r / ldexp(1.0, e - 1)) - 2;
    return (uint8_t)(sign | ((e + 1) << 1) | m);
}

/* E8M0 shared scale: code c means 2^(c-127); 255 is NaN. */
double or_double_from_e8m0(uint8_t c) {
    if (c == 255) return NAN;
    return ldexp(1.0, (int)c - 127);
}

/* MX block quantisation of one block of n (<= 32) values [OCP-MX, conversion
 * to MX formats]: shared_exp = floor(log2(max |v|)) - emax_elem, with
 * emax_elem the exponent of the element format's largest normal (8 for E4M3,
 * 448 = 1.75 * 2^8; 2 for E2M1, 6 = 1.5 * 2^2), clamped to the E8M0 range
 * [-127, 127] (an all-zero block therefore gets code 0); each element is
 * v / 2^shared_exp rounded to the element format (RNE, saturating).  One code
 * per element (E2M1: in the low 4 bits). */
static void or_mx_block_fmt(int fmt, const double* v, int n, uint8_t* codes, uint8_t* scale) {
    const int fp4 = fmt == OR_MXFP4;
    double amax = 0.0;
    for (int i = 0; i < n; ++i) {
        double a = fabs(v[i]);
        if (a > amax) amax = a;
    }
    int se;
    if (amax == 0.0) {
        se = -127;
    } else {
        int e2;
        frexp(amax, &e2);   /* floor(log2(amax)) = e2 - 1 */
        se = (e2 - 1) - (fp4 ? 2 : 8);
        if (se < -127) se = -127;
        if (se > 127) se = 127;
    }
    *scale = (uint8_t)(se + 127);
    for (int i = 0; i < n; ++i)
        codes[i] = fp4 ? or_e2m1_from_double(ldexp(v[i], -se)) : or_e4m3_from_double(ldexp(v[i], -se));
}
static void or_mx_block(const double* v, int n, uint8_t* codes, uint8_t* scale) {
    or_mx_block_fmt(OR_MXFP8, v, n, codes, scale);
}

/* MXFP4 rows hold two E2M1 codes per byte: element 2i in the low 4 bits of
 * byte i, element 2i + 1 in the high 4 bits. */
static inline uint8_t or_fp4_code(const void* row, int64_t i) {
    const uint8_t b = ((const uint8_t*)row)[i >> 1];
    return (uint8_t)((i & 1) ? b >> 4 : b & 0xF);
}
static void or_fp4_pack(const uint8_t* codes, int64_t n, uint8_t* out) {
    for (int64_t j = 0; j < n / 2; ++j) out[j] = (uint8_t)((codes[2 * j] & 0xF) | ((codes[2 * j + 1] & 0xF) << 4));
}

/* Quantise a row-major [rows, cols] float32 matrix to MXFP8 (fmt 2: one code
 * byte per element) or MXFP4 (fmt 3: packed, cols / 2 bytes per row) with
 * blocks of 32 along the columns.  cols must be a multiple of 32. */
int or_mx_quantize_f32_fmt(int fmt, const float* in, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales) {
    if (cols % OR_MX_BLOCK || (fmt != OR_MXFP8 && fmt != OR_MXFP4)) return 1;
    const int64_t nb = cols / OR_MX_BLOCK;
    const int64_t rb = fmt == OR_MXFP4 ? cols / 2 : cols;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double buf[OR_MX_BLOCK];
        uint8_t c[OR_MX_BLOCK];
        for (int64_t b = 0; b < nb; ++b) {
            for (int i = 0; i < OR_MX_BLOCK; ++i) buf[i] = (double)in[r * cols + b * OR_MX_BLOCK + i];
            or_mx_block_fmt(fmt, buf, OR_MX_BLOCK, c, scales + r * nb + b);
            if (fmt == OR_MXFP4) or_fp4_pack(c, OR_MX_BLOCK, codes + r * rb + b * (OR_MX_BLOCK / 2));
            else memcpy(codes + r * rb + b * OR_MX_BLOCK, c, OR_MX_BLOCK);
        }
    }
    return 0;
}
int or_mx_quantize_f32(const float* in, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales) {
    return or_mx_quantize_f32_fmt(OR_MXFP8, in, rows, cols, codes, scales);
}

/* Bulk helpers for the tests. */
void or_bf16_from_double_array(const double* in, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = or_bf16_from_double(in[i]);
}
void or_e4m3_from_double_array(const double* in, uint8_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = or_e4m3_from_double(in[i]);
}
void or_double_from_e4m3_array(const uint8_t* in, double* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = or_double_from_e4m3(in[i]);
}
void or_e2m1_from_double_array(const double* in, uint8_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = or_e2m1_from_double(in[i]);
}

/* Decode element i of a stored row to double.  For MXFP8 and MXFP4 the
 * row's scale array holds one E8M0 code per 32 consecutive elements. */
static inline double or_load(int fmt, const void* row, const uint8_t* scale_row, int64_t i) {
    switch (fmt) {
    case OR_F32: return (double)((const float*)row)[i];
    case OR_BF16: return or_double_from_bf16(((const uint16_t*)row)[i]);
    case OR_MXFP4: return or_double_from_e2m1(or_fp4_code(row, i)) * or_double_from_e8m0(scale_row[i / OR_MX_BLOCK]);
    default:
        return or_double_from_e4m3(((const uint8_t*)row)[i]) * or_double_from_e8m0(scale_row[i / OR_MX_BLOCK]);
    }
}

static inline int or_is_mx(int fmt) { return fmt == OR_MXFP8 || fmt == OR_MXFP4; }
static inline size_t or_elem_bytes(int fmt) { return fmt == OR_F32 ? 4 : (fmt == OR_BF16 ? 2 : 1); }
/* Size in bytes of one stored row of n elements (data only; MXFP4 packs two
 * elements per byte). */
static inline size_t or_row_bytes(int fmt, int64_t n) {
    return fmt == OR_MXFP4 ? (size_t)n / 2 : (size_t)n * or_elem_bytes(fmt);
}

/* Store a row of n doubles in a storage format (MX formats: n % 32 == 0). */
static void or_store_row(int fmt, const double* v, int64_t n, void* row, uint8_t* scale_row) {
    if (fmt == OR_F32) {
        for (int64_t i = 0; i < n; ++i) ((float*)row)[i] = (float)v[i];
    } else if (fmt == OR_BF16) {
        for (int64_t i = 0; i < n; ++i) ((uint16_t*)row)[i] = or_bf16_from_double(v[i]);
    } else if (fmt == OR_MXFP4) {
        uint8_t c[OR_MX_BLOCK];
        for (int64_t b = 0; b < n / OR_MX_BLOCK; ++b) {
            or_mx_block_fmt(OR_MXFP4, v + b * OR_MX_BLOCK, OR_MX_BLOCK, c, scale_row + b);
            or_fp4_pack(c, OR_MX_BLOCK, (uint8_t*)row + b * (OR_MX_BLOCK / 2));
        }
    } else {
        for (int64_t b = 0; b < n / OR_MX_BLOCK; ++b)
            or_mx_block(v + b * OR_MX_BLOCK, OR_MX_BLOCK, (uint8_t*)row + b * OR_MX_BLOCK, scale_row + b);
    }
}

/* Value a stored row holds after or_store_row (the storage round trip). */
static void or_round_trip_row(int fmt, double* v, int64_t n) {
    if (fmt == OR_F32) {
        for (int64_t i = 0; i < n; ++i) v[i] = (double)(float)v[i];
    } else if (fmt == OR_BF16) {
        for (int64_t i = 0; i < n; ++i) v[i] = or_double_from_bf16(or_bf16_from_double(v[i]));
    } else {
        for (int64_t b = 0; b < n / OR_MX_BLOCK; ++b) {
            uint8_t c[OR_MX_BLOCK], s;
            or_mx_block_fmt(fmt, v + b * OR_MX_BLOCK, OR_MX_BLOCK, c, &s);
            for (int i = 0; i < OR_MX_BLOCK; ++i)
                v[b * OR_MX_BLOCK + i] =
                    (fmt == OR_MXFP4 ? or_double_from_e2m1(c[i]) : or_double_from_e4m3(c[i])) * or_double_from_e8m0(s);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* 1. Routing: score function, top-k, normalisation.                        */
/* ------------------------------------------------------------------------ */
/*
 * [TE-EP] the router takes fp32 logits ("logits_2d -> fp32 promotion") and
 * offers both score functions (softmax and sigmoid); the normalised variant
 * divides the selected scores by their sum plus 1e-20 (commit "strip
 * PR-response framing ...; drop sparse_probs NaN sanitizer").
 *
 * Selection works on the logit, which is monotone in both scores.  k passes:
 * each pass takes the largest logit among the experts not yet taken, scanning
 * experts in ascending order and replacing the running best only on a strictly
 * larger logit, so equal logits go to the lower expert index.  Slot j holds the
 * j-th pick.
 *
 * Weights: softmax: p = exp(l - max) / sum_e exp(l_e - max) over all E
 * experts; with renorm, w_j = p_j / (sum_j p_j + 1e-20).  sigmoid:
 * s = 1 / (1 + exp(-l)), w_j = s_j / (sum_j s_j + 1e-20) (always normalised).
 *
 * Optional selection-only expert bias ([TE-EP] commit messages: the router's
 * expert routing bias, "use_expert_routing_bias", with a sigmoid config that
 * uses a strong bias, and a zero bias that collapses to no bias).  The pages
 * give no formula; here the bias b_e shifts the selection key of expert e to
 * the float32 sum key_e = fl32(l_e + b_e), and the k picks are the largest
 * keys (ties to the lower index).  The weights above use the unbiased logits
 * of the picked experts, so the bias changes which experts are chosen, never
 * how the chosen ones are weighted.  bias NULL: key = logit.
 * Returns 0, or 1 on bad sizes.
 */
int or_route_biased(int T, int E, int k, int score, int renorm, const float* logits, const float* bias,
                    int32_t* idx, float* w) {
    if (T < 0 || E <= 0 || k <= 0 || k > E) return 1;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        const float* l = logits + (int64_t)t * E;
        unsigned char* taken = (unsigned char*)calloc((size_t)E, 1);
        float* key = (float*)malloc(sizeof(float) * (size_t)E);
        for (int e = 0; e < E; ++e) key[e] = bias ? (float)(l[e] + bias[e]) : l[e];
        int32_t* sel = idx + (int64_t)t * k;
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || key[e] > key[best]) best = e;
            }
            taken[best] = 1;
            sel[j] = best;
        }
        free(key);
        free(taken);
        double* sc = (double*)malloc(sizeof(double) * (size_t)k);
        double sum_sel = 0.0;
        if (score == OR_SOFTMAX) {
            double m = -INFINITY;
            for (int e = 0; e < E; ++e) if ((double)l[e] > m) m = (double)l[e];
            double Z = 0.0;
            for (int e = 0; e < E; ++e) Z += exp((double)l[e] - m);
            for (int j = 0; j < k; ++j) {
                sc[j] = exp((double)l[sel[j]] - m) / Z;
                sum_sel += sc[j];
            }
            for (int j = 0; j < k; ++j)
                w[(int64_t)t * k + j] = (float)(renorm ? sc[j] / (sum_sel + 1e-20) : sc[j]);
        } else {
            for (int j = 0; j < k; ++j) {
                sc[j] = 1.0 / (1.0 + exp(-(double)l[sel[j]]));
                sum_sel += sc[j];
            }
            for (int j = 0; j < k; ++j) w[(int64_t)t * k + j] = (float)(sc[j] / (sum_sel + 1e-20));
        }
        free(sc);
    }
    return 0;
}

int or_route(int T, int E, int k, int score, int renorm, const float* logits, int32_t* idx, float* w) {
    return or_route_biased(T, E, k, score, renorm, logits, NULL, idx, w);
}

/* ------------------------------------------------------------------------ */
/* 2. Grouping: per-expert counts, aligned offsets, row maps.               */
/* ------------------------------------------------------------------------ */
/*
 * [TE-EP] commit "plumb token_counts to grouped_gemm and zero 0-token wgrad
 * slices": rows are laid out expert-major, [expert_0 | expert_1 | ... | tail],
 * each expert's block zero-padded to the alignment, with the per-expert counts
 * kept on the device and used as the grouped GEMM's group sizes ([ISSUE]: all
 * problem sizes come from device buffers).  [CUDNN] Summary: an expert id of -1
 * is a dropped route.
 *
 * counts[e]     = number of (t, j) with idx[t, j] == e
 * offsets[0]    = 0, offsets[e+1] = offsets[e] + align * ceil(counts[e] / align)
 * row_map[t*k+j]= destination row of route (t, j): routes are placed in
 *                 ascending (t, j) order within their expert's block; -1 for a
 *                 dropped route
 * src_map[row]  = t*k + j for a real row, -1 for padding and the unused tail
 * Ids outside [-1, E), and an id repeated within one token's k slots (top-k
 * never repeats an expert), are treated as dropped and counted in *n_bad.
 * Returns 0, 1 on bad sizes, 2 if R_cap is too small.
 */
int or_group(int T, int E, int k, int align, int64_t R_cap, const int32_t* idx, int32_t* counts,
             int32_t* offsets, int32_t* row_map, int32_t* src_map, int32_t* n_bad) {
    if (T < 0 || E <= 0 || k <= 0 || align <= 0) return 1;
    int32_t bad = 0;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    /* route (t, j) is live when its id is in [0, E) and no earlier slot of
     * token t holds the same id (top-k never repeats an expert; a repeat in a
     * caller's table is dropped and counted like an out-of-range id) */
    unsigned char* live = (unsigned char*)malloc((size_t)T * k + 1);
    for (int64_t i = 0; i < (int64_t)T * k; ++i) {
        int32_t e = idx[i];
        live[i] = 0;
        if (e == -1) continue;
        int dup = 0;
        for (int64_t q = i - i % k; q < i; ++q) dup |= idx[q] == e;
        if (e < -1 || e >= E || dup) { ++bad; continue; }
        live[i] = 1;
        counts[e] += 1;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + ((counts[e] + align - 1) / align) * align;
    if ((int64_t)offsets[E] > R_cap) { free(live); return 2; }
    for (int64_t r = 0; r < R_cap; ++r) src_map[r] = -1;
    int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    for (int e = 0; e < E; ++e) cursor[e] = offsets[e];
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            int64_t i = (int64_t)t * k + j;
            int32_t e = idx[i];
            if (!live[i]) { row_map[i] = -1; continue; }
            int32_t row = cursor[e]++;
            row_map[i] = row;
            src_map[row] = (int32_t)i;
        }
    }
    free(cursor);
    free(live);
    if (n_bad) *n_bad = bad;
    return 0;
}

/* ------------------------------------------------------------------------ */
/* 3. Permute: copy each token's row to its routes' destination rows.       */
/* ------------------------------------------------------------------------ */
/* Xp[row_map[t*k+j]] = x[t], byte for byte; rows [0, n_rows) that receive no
 * route (padding) are zero ([TE-EP] zero-padded expert blocks).  Used for the
 * data and, in MXFP8, separately for the scale rows. */
void or_permute(int T, int k, int64_t n_rows, int64_t row_bytes, const uint8_t* x, const int32_t* row_map,
                uint8_t* xp) {
    memset(xp, 0, (size_t)(n_rows * row_bytes));
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int32_t row = row_map[(int64_t)t * k + j];
            if (row < 0) continue;
            memcpy(xp + (int64_t)row * row_bytes, x + (int64_t)t * row_bytes, (size_t)row_bytes);
        }
}

/* ------------------------------------------------------------------------ */
/* 4-5. Expert FFN of one routed row: gate/up projection, SwiGLU, down.     */
/* ------------------------------------------------------------------------ */
/*
 * [CUDNN] Summary: local experts compute silu(gate) * up; [BLOCK] Diagram:
 * grouped GEMM fused with SwiGLU, then the down projection.  The weights have
 * logical shapes fc1 (E, H, 2F) with gate = columns [0, F) and up = columns
 * [F, 2F), and fc2 (E, F, H) ([CUDNN] MoeEp.__call__ docstring).  They are
 * stored K-contiguous: W1s[e][n][h] = fc1[e][h][n] and W2s[e][h][f] =
 * fc2[e][f][h].
 *
 * g_f = sum_h x[h] * W1s[e][f][h],  u_f = sum_h x[h] * W1s[e][F+f][h]
 * h_f = store_h( silu(g_f) * u_f ),  silu(g) = g / (1 + exp(-g))
 * Yp_o = store_out( sum_f h_f * W2s[e][o][f] )   (uses the stored h)
 * stash = store_stash(g), store_stash(u)     (backward's saved activations)
 *
 * Placement of the routing weight w of the row ([CUDNN] Summary: the router
 * weight is applied in the FC1 or the FC2 epilogue; [TE-EP] commits: the
 * weights may be applied early, before the combine).  site OR_AT_COMBINE
 * leaves the row unweighted (the combine applies w).  OR_AT_FC1 scales the
 * SwiGLU output before it is stored, h_f = store_h( w * silu(g_f) * u_f ).
 * OR_AT_FC2 scales the down projection before it is stored,
 * Yp_o = store_out( w * sum_f h_f W2s[e][o][f] ).  In exact arithmetic all
 * three give the same combined y; only the rounding points differ.
 *
 * fmt is the storage format of x and the weights, h_fmt that of h (F32, BF16 or
 * MXFP8 with blocks along F), y_fmt that of Yp and y (F32 or BF16), s_fmt that
 * of the stash (F32 or BF16).  Any output pointer may be NULL.
 */
void or_expert_row(int H, int F, int fmt, const void* x_row, const uint8_t* x_scale_row, const void* w1_e,
                   const uint8_t* w1s_e, const void* w2_e, const uint8_t* w2s_e, int h_fmt, int y_fmt, int s_fmt,
                   int site, double row_w, void* h_out, uint8_t* h_scale_out, void* yp_out, void* stash_out) {
    double* xv = (double*)malloc(sizeof(double) * (size_t)H);
    double* hv = (double*)malloc(sizeof(double) * (size_t)F);
    double* gu = (double*)malloc(sizeof(double) * 2 * (size_t)F);
    for (int h = 0; h < H; ++h) xv[h] = or_load(fmt, x_row, x_scale_row, h);
    for (int n = 0; n < 2 * F; ++n) {
        const void* wrow = (const uint8_t*)w1_e + (size_t)n * or_row_bytes(fmt, H);
        const uint8_t* wsrow = or_is_mx(fmt) ? w1s_e + (size_t)n * (H / OR_MX_BLOCK) : NULL;
        double acc = 0.0;
        for (int h = 0; h < H; ++h) acc += xv[h] * or_load(fmt, wrow, wsrow, h);
        gu[n] = acc;
    }
    for (int f = 0; f < F; ++f) {
        double g = gu[f], u = gu[F + f];
        hv[f] = or_swiglu(g, u);
        if (site == OR_AT_FC1) hv[f] *= row_w;
    }
    if (stash_out) or_store_row(s_fmt, gu, 2 * F, stash_out, NULL);
    if (h_out) or_store_row(h_fmt, hv, F, h_out, h_scale_out);
    or_round_trip_row(h_fmt, hv, F); /* the down projection reads the stored h */
    if (yp_out) {
        double* yv = (double*)malloc(sizeof(double) * (size_t)H);
        for (int o = 0; o < H; ++o) {
            const void* wrow = (const uint8_t*)w2_e + (size_t)o * or_row_bytes(fmt, F);
            const uint8_t* wsrow = or_is_mx(fmt) ? w2s_e + (size_t)o * (F / OR_MX_BLOCK) : NULL;
            double acc = 0.0;
            for (int f = 0; f < F; ++f) acc += hv[f] * or_load(fmt, wrow, wsrow, f);
            yv[o] = site == OR_AT_FC2 ? row_w * acc : acc;
        }
        or_store_row(y_fmt, yv, H, yp_out, NULL);
        free(yv);
    }
    free(xv);
    free(hv);
    free(gu);
}


/* ------------------------------------------------------------------------ */
/* Forward for a list of tokens (per-token evaluation, no permutation).     */
/* ------------------------------------------------------------------------ */
/*
 * For each listed token t and slot j with e = idx[t, j] != -1, evaluates the
 * expert FFN on x[t] (the same bytes the permuted row holds) and writes, at
 * position (i, j) of the outputs (i = position of t in the list):
 *   h_out[i*k+j]  (F elements, h_fmt; MXFP8 scales in h_scale_out)
 *   yp_out[i*k+j] (H elements, y_fmt)
 *   stash_out[i*k+j] (2F elements, s_fmt)
 * and the combine ([CUDNN] Summary, per-top-k combine; [TE-EP] expert outputs
 * summed across the top-k):
 *   y_out[i] = store_y( sum_{j ascending, idx != -1} c(t, j) * Yp(t, j) )
 * accumulated in double from the stored Yp, with c = w[t, j] for site
 * OR_AT_COMBINE and c = 1 when the weight was applied in an epilogue (the row
 * of (t, j) then carries w[t, j], see or_expert_row).  Any output may be NULL.
 */
int or_forward_tokens(int H, int F, int k, int fmt, int h_fmt, int y_fmt, int s_fmt, int site, int n_tok,
                      const int32_t* tokens, const void* x, const uint8_t* x_scale, const void* w1,
                      const uint8_t* w1_scale, const void* w2, const uint8_t* w2_scale, const int32_t* idx,
                      const float* w, void* h_out, uint8_t* h_scale_out, void* yp_out, void* stash_out,
                      void* y_out) {
    if (or_is_mx(fmt) && (H % OR_MX_BLOCK || F % OR_MX_BLOCK)) return 1;
    if (or_is_mx(h_fmt) && F % OR_MX_BLOCK) return 1;
    const size_t w1_expert = (size_t)2 * F * or_row_bytes(fmt, H), w2_expert = (size_t)H * or_row_bytes(fmt, F);
    const size_t w1s_expert = (size_t)2 * F * (H / OR_MX_BLOCK), w2s_expert = (size_t)H * (F / OR_MX_BLOCK);
    const size_t hb = or_row_bytes(h_fmt, F), yb = or_row_bytes(y_fmt, H), sb = or_row_bytes(s_fmt, 2 * F);
    const int64_t hsb = or_is_mx(h_fmt) ? F / OR_MX_BLOCK : 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ij = 0; ij < (int64_t)n_tok * k; ++ij) {
        const int64_t i = ij / k;
        const int j = (int)(ij % k);
        const int64_t t = tokens[i];
        const int32_t e = idx[t * k + j];
        if (e < 0) continue;
        const void* xr = (const uint8_t*)x + (size_t)t * or_row_bytes(fmt, H);
        const uint8_t* xs = or_is_mx(fmt) ? x_scale + (size_t)t * (H / OR_MX_BLOCK) : NULL;
        or_expert_row(H, F, fmt, xr, xs, (const uint8_t*)w1 + e * w1_expert,
                      or_is_mx(fmt) ? w1_scale + e * w1s_expert : NULL, (const uint8_t*)w2 + e * w2_expert,
                      or_is_mx(fmt) ? w2_scale + e * w2s_expert : NULL, h_fmt, y_fmt, s_fmt, site,
                      (double)w[t * k + j],
                      h_out ? (uint8_t*)h_out + ij * hb : NULL, h_scale_out ? h_scale_out + ij * hsb : NULL,
                      (uint8_t*)yp_out + ij * yb, stash_out ? (uint8_t*)stash_out + ij * sb : NULL);
    }
    if (y_out) {
        const size_t ob = or_elem_bytes(y_fmt);
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < n_tok; ++i) {
            const int64_t t = tokens[i];
            double* acc = (double*)calloc((size_t)H, sizeof(double));
            for (int j = 0; j < k; ++j) {
                if (idx[t * k + j] < 0) continue;
                const void* yr = (const uint8_t*)yp_out + (i * k + j) * yb;
                const double wt = site == OR_AT_COMBINE ? (double)w[t * k + j] : 1.0;
                for (int o = 0; o < H; ++o) acc[o] += wt * or_load(y_fmt, yr, NULL, o);
            }
            or_store_row(y_fmt, acc, H, (uint8_t*)y_out + i * H * ob, NULL);
            free(acc);
        }
    }
    return 0;
}

/* Combine of already-permuted expert outputs ([CUDNN] per-top-k combine):
 * y[t] = store_y( sum_{j ascending} w[t,j] * Yp[row_map[t*k+j]] ), skipping
 * dropped routes.  Rows that no route maps are never read.  w NULL: the
 * weights were applied in an expert epilogue and the routes are summed. */
void or_combine(int T, int H, int k, int y_fmt, const void* yp, const int32_t* row_map, const float* w, void* y) {
    const size_t ob = or_elem_bytes(y_fmt);
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        double* acc = (double*)calloc((size_t)H, sizeof(double));
        for (int j = 0; j < k; ++j) {
            int32_t row = row_map[(int64_t)t * k + j];
            if (row < 0) continue;
            const void* yr = (const uint8_t*)yp + (size_t)row * H * ob;
            const double wt = w ? (double)w[(int64_t)t * k + j] : 1.0;
            for (int o = 0; o < H; ++o) acc[o] += wt * or_load(y_fmt, yr, NULL, o);
        }
        or_store_row(y_fmt, acc, H, (uint8_t*)y + (size_t)t * H * ob, NULL);
        free(acc);
    }
}

/* ------------------------------------------------------------------------ */
/* Backward of the expert FFN and the combine (training workload).          */
/* ------------------------------------------------------------------------ */
/*
 * [TE-EP] commit "plumb token_counts ... zero 0-token wgrad slices": the
 * weight gradient of an expert that received no rows is zero.  [CUDNN]
 * Summary: backward re-dispatches the output gradient along the forward routes
 * and recomputes SwiGLU from the saved pre-activation stash (here the stored g
 * and u), and [TE-EP] keeps d_x in x's dtype.
 *
 * With the forward's stored h, stash (g|u) and routing state:
 *   dYp[row]    = store_g( w[t,j] * dY[t] )                  (b1)
 *   dH[row, f]  = sum_o dYp[row, o] * W2s[e][o][f]           (b2)
 *   sig = 1/(1+exp(-g)),  silu = g*sig
 *   dG = dH * u * sig * (1 + g*(1-sig)),  dU = dH * silu(g)
 *   dGU[row]    = store_g( dG | dU )                          (2F columns)
 *   dW2s[e][o][f] = sum_{rows of e, ascending} h[row, f] * dYp[row, o]   (b3)
 *   dXp[row, c] = store_g( sum_n dGU[row, n] * W1s[e][n][c] ) (b4)
 *   dW1s[e][n][c] = sum_{rows of e, ascending} dGU[row, n] * Xp[row, c] (b5)
 *   dX[t]       = store_g( sum_{j ascending} dXp[row_map[t,j]] )          (b6)
 * dW1s / dW2s are float32 in the stored (K-contiguous) weight layout and are
 * exactly 0 for an expert with no rows.  g_fmt is the gradient storage format
 * (x's format: F32 or BF16).  The routing weights are treated as constants
 * (their gradient is not part of this path).
 */
int or_backward(int T, int H, int F, int E, int k, int fmt, int g_fmt, const void* x, const void* w1,
                const void* w2, const float* w, const int32_t* row_map, const int32_t* src_map,
                const int32_t* offsets, const void* h_saved, int h_fmt, const void* stash, int s_fmt,
                const void* dy, void* dyp, void* dgu, void* dxp, void* dx, float* dw1, float* dw2) {
    if (or_is_mx(fmt) || or_is_mx(h_fmt)) return 1;
    const size_t eb = or_elem_bytes(fmt), gb = or_elem_bytes(g_fmt);
    const size_t hb = or_row_bytes(h_fmt, F), sb = or_row_bytes(s_fmt, 2 * F);
    const int64_t R = offsets[E];
    /* b1 */
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        double* v = (double*)malloc(sizeof(double) * (size_t)H);
        int32_t s = src_map[r];
        if (s < 0) {
            for (int o = 0; o < H; ++o) v[o] = 0.0;
        } else {
            int64_t t = s / k;
            for (int o = 0; o < H; ++o) v[o] = (double)w[s] * or_load(g_fmt, (const uint8_t*)dy + t * H * gb, NULL, o);
        }
        or_store_row(g_fmt, v, H, (uint8_t*)dyp + r * H * gb, NULL);
        free(v);
    }
    /* b2 + dSwiGLU, b4 */
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < R; ++r) {
        int e = 0;
        while (offsets[e + 1] <= r) ++e;
        double* dh = (double*)malloc(sizeof(double) * (size_t)F);
        double* d = (double*)malloc(sizeof(double) * 2 * (size_t)F);
        double* dxr = (double*)malloc(sizeof(double) * (size_t)H);
        const void* dyr = (const uint8_t*)dyp + r * H * gb;
        const uint8_t* w2e = (const uint8_t*)w2 + (size_t)e * H * F * eb;
        for (int f = 0; f < F; ++f) dh[f] = 0.0;
        for (int o = 0; o < H; ++o) {
            double a = or_load(g_fmt, dyr, NULL, o);
            const void* wrow = w2e + (size_t)o * F * eb;
            for (int f = 0; f < F; ++f) dh[f] += a * or_load(fmt, wrow, NULL, f);
        }
        const void* sr = (const uint8_t*)stash + r * sb;
        for (int f = 0; f < F; ++f) {
            double g = or_load(s_fmt, sr, NULL, f), u = or_load(s_fmt, sr, NULL, F + f), dg, du;
            or_swiglu_grad(g, u, &dg, &du);
            d[f] = dh[f] * dg;
            d[F + f] = dh[f] * du;
        }
        void* dgr = (uint8_t*)dgu + r * 2 * F * gb;
        or_store_row(g_fmt, d, 2 * F, dgr, NULL);
        const uint8_t* w1e = (const uint8_t*)w1 + (size_t)e * 2 * F * H * eb;
        for (int c = 0; c < H; ++c) dxr[c] = 0.0;
        for (int n = 0; n < 2 * F; ++n) {
            double a = or_load(g_fmt, dgr, NULL, n);
            const void* wrow = w1e + (size_t)n * H * eb;
            for (int c = 0; c < H; ++c) dxr[c] += a * or_load(fmt, wrow, NULL, c);
        }
        or_store_row(g_fmt, dxr, H, (uint8_t*)dxp + r * H * gb, NULL);
        free(dh);
        free(d);
        free(dxr);
    }
    /* b3, b5 */
#pragma omp parallel for schedule(dynamic, 1)
    for (int e = 0; e < E; ++e) {
        float* w2g = dw2 + (size_t)e * H * F;
        float* w1g = dw1 + (size_t)e * 2 * F * H;
        double* acc2 = (double*)calloc((size_t)H * F, sizeof(double));
        double* acc1 = (double*)calloc((size_t)2 * F * H, sizeof(double));
        for (int64_t r = offsets[e]; r < offsets[e + 1]; ++r) {
            int32_t s = src_map[r];
            const void* hr = (const uint8_t*)h_saved + r * hb;
            const void* dyr = (const uint8_t*)dyp + r * H * gb;
            for (int o = 0; o < H; ++o) {
                double a = or_load(g_fmt, dyr, NULL, o);
                for (int f = 0; f < F; ++f) acc2[(size_t)o * F + f] += or_load(h_fmt, hr, NULL, f) * a;
            }
            if (s < 0) continue; /* padding rows of Xp are zero */
            const void* xr = (const uint8_t*)x + (size_t)(s / k) * H * eb;
            const void* dgr = (const uint8_t*)dgu + r * 2 * F * gb;
            for (int n = 0; n < 2 * F; ++n) {
                double a = or_load(g_fmt, dgr, NULL, n);
                for (int c = 0; c < H; ++c) acc1[(size_t)n * H + c] += a * or_load(fmt, xr, NULL, c);
            }
        }
        for (size_t i = 0; i < (size_t)H * F; ++i) w2g[i] = (float)acc2[i];
        for (size_t i = 0; i < (size_t)2 * F * H; ++i) w1g[i] = (float)acc1[i];
        free(acc2);
        free(acc1);
    }
    /* b6 */
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        double* v = (double*)calloc((size_t)H, sizeof(double));
        for (int j = 0; j < k; ++j) {
            int32_t r = row_map[(int64_t)t * k + j];
            if (r < 0) continue;
            for (int c = 0; c < H; ++c) v[c] += or_load(g_fmt, (const uint8_t*)dxp + (size_t)r * H * gb, NULL, c);
        }
        or_store_row(g_fmt, v, H, (uint8_t*)dx + (size_t)t * H * gb, NULL);
        free(v);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Sampled backward quantities at full size (computed one by one).          */
/* ------------------------------------------------------------------------ */
/* Forward pre-activations of one route, recomputed from x: g (F) and u (F)
 * rounded to the stash format, and h rounded to h_fmt. */
static void or_route_gu(int H, int F, int fmt, int s_fmt, int h_fmt, const void* x_row, const void* w1_e,
                        double* g, double* u, double* h) {
    const size_t eb = or_elem_bytes(fmt);
    double* xv = (double*)malloc(sizeof(double) * (size_t)H);
    double* gu = (double*)malloc(sizeof(double) * 2 * (size_t)F);
    for (int c = 0; c < H; ++c) xv[c] = or_load(fmt, x_row, NULL, c);
    for (int n = 0; n < 2 * F; ++n) {
        const void* wrow = (const uint8_t*)w1_e + (size_t)n * H * eb;
        double acc = 0.0;
        for (int c = 0; c < H; ++c) acc += xv[c] * or_load(fmt, wrow, NULL, c);
        gu[n] = acc;
    }
    for (int f = 0; f < F; ++f) h[f] = or_swiglu(gu[f], gu[F + f]);
    or_round_trip_row(h_fmt, h, F);
    or_round_trip_row(s_fmt, gu, 2 * F);
    for (int f = 0; f < F; ++f) { g[f] = gu[f]; u[f] = gu[F + f]; }
    free(xv);
    free(gu);
}

/* dX rows of the listed tokens (b1, b2, dSwiGLU, b4, b6 along one token's
 * routes).  dx_out is [n_tok, H] in g_fmt. */
int or_backward_dx_tokens(int H, int F, int k, int fmt, int g_fmt, int h_fmt, int s_fmt, int n_tok,
                          const int32_t* tokens, const void* x, const void* w1, const void* w2,
                          const int32_t* idx, const float* w, const void* dy, void* dx_out) {
    if (or_is_mx(fmt)) return 1;
    const size_t eb = or_elem_bytes(fmt), gb = or_elem_bytes(g_fmt);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_tok; ++i) {
        const int64_t t = tokens[i];
        double* g = (double*)malloc(sizeof(double) * (size_t)F);
        double* u = (double*)malloc(sizeof(double) * (size_t)F);
        double* hh = (double*)malloc(sizeof(double) * (size_t)F);
        double* dyp = (double*)malloc(sizeof(double) * (size_t)H);
        double* dh = (double*)malloc(sizeof(double) * (size_t)F);
        double* d = (double*)malloc(sizeof(double) * 2 * (size_t)F);
        double* dxr = (double*)malloc(sizeof(double) * (size_t)H);
        double* acc = (double*)calloc((size_t)H, sizeof(double));
        const void* xr = (const uint8_t*)x + (size_t)t * H * eb;
        for (int j = 0; j < k; ++j) {
            int32_t e = idx[t * k + j];
            if (e < 0) continue;
            const uint8_t* w1e = (const uint8_t*)w1 + (size_t)e * 2 * F * H * eb;
            const uint8_t* w2e = (const uint8_t*)w2 + (size_t)e * H * F * eb;
            or_route_gu(H, F, fmt, s_fmt, h_fmt, xr, w1e, g, u, hh);
            for (int o = 0; o < H; ++o)
                dyp[o] = (double)w[t * k + j] * or_load(g_fmt, (const uint8_t*)dy + t * H * gb, NULL, o);
            or_round_trip_row(g_fmt, dyp, H);
            for (int f = 0; f < F; ++f) dh[f] = 0.0;
            for (int o = 0; o < H; ++o) {
                const void* wrow = w2e + (size_t)o * F * eb;
                for (int f = 0; f < F; ++f) dh[f] += dyp[o] * or_load(fmt, wrow, NULL, f);
            }
            for (int f = 0; f < F; ++f) {
                double dg, du;
                or_swiglu_grad(g[f], u[f], &dg, &du);
                d[f] = dh[f] * dg;
                d[F + f] = dh[f] * du;
            }
            or_round_trip_row(g_fmt, d, 2 * F);
            for (int c = 0; c < H; ++c) dxr[c] = 0.0;
            for (int n = 0; n < 2 * F; ++n) {
                const void* wrow = w1e + (size_t)n * H * eb;
                for (int c = 0; c < H; ++c) dxr[c] += d[n] * or_load(fmt, wrow, NULL, c);
            }
            or_round_trip_row(g_fmt, dxr, H);
            for (int c = 0; c < H; ++c) acc[c] += dxr[c];
        }
        or_store_row(g_fmt, acc, H, (uint8_t*)dx_out + (size_t)i * H * gb, NULL);
        free(g); free(u); free(hh); free(dyp); free(dh); free(d); free(dxr); free(acc);
    }
    return 0;
}

/* Selected entries of dW2s[e] and dW1s[e] for one expert e, recomputing each
 * of the expert's routes from x (rows in ascending order, as listed by
 * src_map over [offsets[e], offsets[e+1])).
 *   dw2_out[i] = dW2s[e][o2[i]][f2[i]]   for i < n2
 *   dw1_out[i] = dW1s[e][n1[i]][c1[i]]   for i < n1          */
int or_backward_dw_entries(int H, int F, int k, int fmt, int g_fmt, int h_fmt, int s_fmt, int e,
                           const void* x, const void* w1, const void* w2, const float* w, const int32_t* src_map,
                           const int32_t* offsets, const void* dy, int n2, const int32_t* o2, const int32_t* f2,
                           double* dw2_out, int n1, const int32_t* n1i, const int32_t* c1, double* dw1_out) {
    if (or_is_mx(fmt)) return 1;
    const size_t eb = or_elem_bytes(fmt), gb = or_elem_bytes(g_fmt);
    const int64_t r0 = offsets[e], r1 = offsets[e + 1];
    const uint8_t* w1e = (const uint8_t*)w1 + (size_t)e * 2 * F * H * eb;
    const uint8_t* w2e = (const uint8_t*)w2 + (size_t)e * H * F * eb;
    for (int i = 0; i < n2; ++i) dw2_out[i] = 0.0;
    for (int i = 0; i < n1; ++i) dw1_out[i] = 0.0;
    const int64_t nr = r1 - r0;
    /* per-row contributions, then summed in ascending row order */
    double* c2 = (double*)calloc((size_t)(nr * (n2 > 0 ? n2 : 1)), sizeof(double));
    double* cc1 = (double*)calloc((size_t)(nr * (n1 > 0 ? n1 : 1)), sizeof(double));
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t q = 0; q < nr; ++q) {
        const int32_t s = src_map[r0 + q];
        if (s < 0) continue; /* padding rows carry zero gradients and zero h */
        const int64_t t = s / k;
        double* g = (double*)malloc(sizeof(double) * (size_t)F);
        double* u = (double*)malloc(sizeof(double) * (size_t)F);
        double* hh = (double*)malloc(sizeof(double) * (size_t)F);
        double* dyp = (double*)malloc(sizeof(double) * (size_t)H);
        const void* xr = (const uint8_t*)x + (size_t)t * H * eb;
        or_route_gu(H, F, fmt, s_fmt, h_fmt, xr, w1e, g, u, hh);
        for (int o = 0; o < H; ++o)
            dyp[o] = (double)w[s] * or_load(g_fmt, (const uint8_t*)dy + t * H * gb, NULL, o);
        or_round_trip_row(g_fmt, dyp, H);
        for (int i = 0; i < n2; ++i) c2[q * n2 + i] = hh[f2[i]] * dyp[o2[i]];
        for (int i = 0; i < n1; ++i) {
            const int n = n1i[i], f = n % F;
            double dh = 0.0;
            for (int o = 0; o < H; ++o) dh += dyp[o] * or_load(fmt, w2e + (size_t)o * F * eb, NULL, f);
            double dg, du;
            or_swiglu_grad(g[f], u[f], &dg, &du);
            double d = n < F ? dh * dg : dh * du;
            d = g_fmt == OR_F32 ? (double)(float)d : or_double_from_bf16(or_bf16_from_double(d));
            cc1[q * n1 + i] = d * or_load(fmt, xr, NULL, c1[i]);
        }
        free(g); free(u); free(hh); free(dyp);
    }
    for (int64_t q = 0; q < nr; ++q) {
        for (int i = 0; i < n2; ++i) dw2_out[i] += c2[q * n2 + i];
        for (int i = 0; i < n1; ++i) dw1_out[i] += cc1[q * n1 + i];
    }
    free(c2);
    free(cc1);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Bulk forms of the per-element steps, for the expert-major front end of   */
/* oracle.py (whose sums over H and F are float64 matrix products).  Each   */
/* applies the single definition above to every element or row.            */
/* ------------------------------------------------------------------------ */
/* h[r][f] = or_swiglu(gu[r][f], gu[r][F + f]) * (rw ? rw[r] : 1), the FC1
 * placement of the routing weight included (see or_expert_row). */
void or_swiglu_rows(const double* gu, int64_t rows, int F, const double* rw, double* h) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int f = 0; f < F; ++f) {
            double v = or_swiglu(gu[r * 2 * F + f], gu[r * 2 * F + F + f]);
            h[r * F + f] = rw ? v * rw[r] : v;
        }
}

/* dgu[r] = dh[r] * dh/dg | dh[r] * dh/du at the stored (g, u) of row r. */
void or_swiglu_grad_rows(const double* gu, const double* dh, int64_t rows, int F, double* dgu) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int f = 0; f < F; ++f) {
            double dg, du;
            or_swiglu_grad(gu[r * 2 * F + f], gu[r * 2 * F + F + f], &dg, &du);
            dgu[r * 2 * F + f] = dh[r * F + f] * dg;
            dgu[r * 2 * F + F + f] = dh[r * F + f] * du;
        }
}

/* Rows of n doubles stored in a format (or_store_row per row). */
void or_store_rows(int fmt, const double* v, int64_t rows, int64_t n, void* out, uint8_t* scale_out) {
    const size_t rb = or_row_bytes(fmt, n);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        or_store_row(fmt, v + r * n, n, (uint8_t*)out + r * rb,
                     or_is_mx(fmt) ? scale_out + r * (n / OR_MX_BLOCK) : NULL);
}

/* Rows of n stored values decoded to double: or_load per element, with the
 * E4M3 decoder tabulated over its 256 codes first for MXFP8. */
void or_decode_rows(int fmt, const void* in, const uint8_t* scale_in, int64_t rows, int64_t n, double* out) {
    const size_t rb = or_row_bytes(fmt, n);
    if (fmt == OR_MXFP8) {
        double tab[256];
        for (int c = 0; c < 256; ++c) tab[c] = or_double_from_e4m3((uint8_t)c);
#pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < rows; ++r) {
            const uint8_t* row = (const uint8_t*)in + r * rb;
            const uint8_t* srow = scale_in + r * (n / OR_MX_BLOCK);
            for (int64_t b = 0; b < n / OR_MX_BLOCK; ++b) {
                const double sc = or_double_from_e8m0(srow[b]);
                for (int i = 0; i < OR_MX_BLOCK; ++i)
                    out[r * n + b * OR_MX_BLOCK + i] = tab[row[b * OR_MX_BLOCK + i]] * sc;
            }
        }
        return;
    }
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const void* row = (const uint8_t*)in + r * rb;
        const uint8_t* srow = fmt == OR_MXFP4 ? scale_in + r * (n / OR_MX_BLOCK) : NULL;
        for (int64_t i = 0; i < n; ++i) out[r * n + i] = or_load(fmt, row, srow, i);
    }
}

int or_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
