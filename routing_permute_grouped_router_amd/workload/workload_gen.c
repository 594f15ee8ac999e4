/*
 * workload_gen.c -- seeded synthetic inputs for the MoE FFN workloads.
 *
 * Holds no step of the MoE method: it only draws Gaussian numbers and stores
 * them as float32, bfloat16 or float64.  Both the GPU path's tests/benchmark
 * and the CPU oracle's tests take their inputs from here.
 *
 * Generator: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
 * numbers: as easy as 1, 2, 3", SC'11), a counter-based generator, so any
 * element can be produced independently of the others.  Counter =
 * (pair index low 32 bits, pair index high 32 bits, tensor id, 0), key = the
 * 64-bit workload seed.  Each counter gives two 53-bit uniforms u1 in (0, 1]
 * and u2 in [0, 1); the Box-Muller transform turns them into two standard
 * normals z0 = r cos(2 pi u2), z1 = r sin(2 pi u2), r = sqrt(-2 ln u1), which
 * become elements 2i and 2i+1 of the tensor's stream.
 *
 * Stored values: f32 = (float)(std * z) (round to nearest even); bf16 = the
 * f32 value rounded to nearest even to bfloat16; f64 = std * z.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

void wl_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        uint64_t p0 = (uint64_t)PHILOX_M0 * c0;
        uint64_t p1 = (uint64_t)PHILOX_M1 * c2;
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += PHILOX_W0;
        k1 += PHILOX_W1;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

static inline void wl_pair(uint64_t seed, uint32_t tensor, uint64_t pair, double* z0, double* z1) {
    const uint32_t ctr[4] = {(uint32_t)pair, (uint32_t)(pair >> 32), tensor, 0u};
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t r[4];
    wl_philox4x32_10(ctr, key, r);
    const uint64_t a = (((uint64_t)r[1] << 32) | r[0]) >> 11;
    const uint64_t b = (((uint64_t)r[3] << 32) | r[2]) >> 11;
    const double u1 = ((double)a + 1.0) * 0x1.0p-53; /* (0, 1] */
    const double u2 = (double)b * 0x1.0p-53;         /* [0, 1) */
    const double rad = sqrt(-2.0 * log(u1));
    const double th = 6.283185307179586476925286766559 * u2;
    *z0 = rad * cos(th);
    *z1 = rad * sin(th);
}

static inline uint16_t wl_bf16_of_f32(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u); /* finite inputs only */
    return (uint16_t)(u >> 16);
}

enum { WL_F32 = 0, WL_BF16 = 1, WL_F64 = 2 };

static inline void wl_store(int kind, void* out, int64_t i, double v) {
    if (kind == WL_F32) ((float*)out)[i] = (float)v;
    else if (kind == WL_BF16) ((uint16_t*)out)[i] = wl_bf16_of_f32((float)v);
    else ((double*)out)[i] = v;
}

/* Elements [start, start + n) of tensor `tensor`'s stream, scaled by std. */
void wl_normal(uint64_t seed, uint32_t tensor, uint64_t start, int64_t n, double std, int kind, void* out) {
    if (n <= 0) return;
    const int64_t chunk = 1 << 16;
    const int64_t nchunks = (n + chunk - 1) / chunk;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < nchunks; ++c) {
        const int64_t lo = c * chunk;
        const int64_t hi = lo + chunk < n ? lo + chunk : n;
        int64_t i = lo;
        while (i < hi) {
            const uint64_t g = start + (uint64_t)i; /* global element index */
            double z0, z1;
            wl_pair(seed, tensor, g >> 1, &z0, &z1);
            if (g & 1u) {
                wl_store(kind, out, i, std * z1);
                i += 1;
            } else {
                wl_store(kind, out, i, std * z0);
                if (i + 1 < hi) wl_store(kind, out, i + 1, std * z1);
                i += 2;
            }
        }
    }
}

int wl_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
