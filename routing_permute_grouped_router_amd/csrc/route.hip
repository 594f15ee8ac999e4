// Routing: score function + top-k + normalisation.
//
// Follows the fp32 router with softmax / sigmoid scores and the
// "sum of selected + 1e-20" normalisation described on the TransformerEngine
// page "[JAX] Expert Parallelism: JAX primitives + VJPs" (commit messages on
// the router), and the routing step of the cudnn-frontend page "Add MoE +
// expert-parallel Python API surface, PyTorch reference, and tests" (Summary).
//
// A token is handled by a group of L lanes (L a power of two, the smallest
// with E <= 32 L), lane r of the group holding the VPL logits of experts
// r VPL .. r VPL + VPL - 1 (VPL = 8, 16 or 32, loaded 16 bytes at a time when
// E % 4 == 0); a wavefront takes 64 / L tokens at once.  With E <= 32 a lane
// is a whole token and no lane exchange happens; with E = 128 four lanes
// share a token and exchange within their quad.  The k
// selections are k group-wide arg-max reductions over (logit desc, expert asc)
// among the experts not yet taken, so equal logits resolve to the lower
// expert index and slot j holds the j-th largest; every lane of the group
// sees every pick, keeps it (KMAX slots), and the normalising sums are
// formed in the same order by all of them.  Lane r writes the picks j with
// j % L == r.
#include "moe_internal.h"

namespace moe {
namespace {

__device__ __forceinline__ bool better(float v, int e, float bv, int be) {
    return v > bv || (v == bv && e < be);
}

template <int L, int VPL, int KMAX>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                    int score, int renorm, int32_t* __restrict__ idx,
                                                    float* __restrict__ w) {
    constexpr int TPW = kWave / L;  // tokens per wavefront
    const int lane = threadIdx.x & 63;
    const int r = lane % L;
    const int64_t t = ((int64_t)blockIdx.x * (256 / kWave) + (threadIdx.x >> 6)) * TPW + lane / L;
    const bool live = t < T;
    const float* row = logits + (live ? t : 0) * (int64_t)E;

    float v[VPL];
    uint32_t avail = 0;
    if (E % 4 == 0) {  // rows are 16-byte aligned: whole float4 of experts
#pragma unroll
        for (int i = 0; i < VPL; i += 4) {
            const int e = r * VPL + i;
            const bool ok = live && e < E;  // e % 4 == 0 and E % 4 == 0: all four or none
            const float4 q = ok ? *(const float4*)(row + e) : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
            v[i] = q.x;
            v[i + 1] = q.y;
            v[i + 2] = q.z;
            v[i + 3] = q.w;
            avail |= ok ? 0xfu << i : 0u;
        }
    } else {
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int e = r * VPL + i;
            const bool ok = live && e < E;
            v[i] = ok ? row[e] : -INFINITY;
            avail |= ok ? 1u << i : 0u;
        }
    }
    // group-wide reductions (the L lanes of a group are consecutive and
    // aligned, so xor offsets below L stay inside it)
    auto gmax = [&](float x) {
#pragma unroll
        for (int off = L / 2; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, kWave));
        return x;
    };
    auto gsum = [&](float x) {
#pragma unroll
        for (int off = L / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, kWave);
        return x;
    };

    float pv[KMAX];
    int pe[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        pv[j] = -INFINITY;
        pe[j] = -1;
        if (j >= k) continue;
        float bv = -INFINITY;
        int be = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int e = r * VPL + i;
            if ((avail >> i & 1) && better(v[i], e, bv, be)) {
                bv = v[i];
                be = e;
            }
        }
#pragma unroll
        for (int off = L / 2; off > 0; off >>= 1) {
            const float ov = __shfl_xor(bv, off, kWave);
            const int oe = __shfl_xor(be, off, kWave);
            if (better(ov, oe, bv, be)) {
                bv = ov;
                be = oe;
            }
        }
        if (be / VPL == r) avail &= ~(1u << (be % VPL));  // the owning lane retires the pick
        pv[j] = bv;
        pe[j] = be;
    }

    float wt[KMAX];
    if (score == MOE_SOFTMAX && !renorm) {
        const float m = pv[0];  // the first pick is the maximum
        float z = 0.f;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            if (r * VPL + i < E) z += expf(v[i] - m);
        z = gsum(z);
#pragma unroll
        for (int j = 0; j < KMAX; ++j) wt[j] = j < k ? expf(pv[j] - m) / z : 0.f;
    } else if (score == MOE_SOFTMAX) {
        // p_j / (sum of the chosen p + 1e-20) with p the softmax over all E:
        // the softmax's normaliser cancels, and the 1e-20 changes nothing in
        // float32 (the sum of the chosen p is at least 1 / E >= 2^-10, whose
        // half ulp 2^-34 exceeds 1e-20), so only the chosen k exponentials
        // are formed.
        const float m = pv[0];
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            wt[j] = j < k ? expf(pv[j] - m) : 0.f;
            s += wt[j];
        }
#pragma unroll
        for (int j = 0; j < KMAX; ++j) wt[j] = wt[j] / s;
    } else {
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            wt[j] = j < k ? 1.0f / (1.0f + expf(-pv[j])) : 0.f;
            s += wt[j];
        }
#pragma unroll
        for (int j = 0; j < KMAX; ++j) wt[j] = wt[j] / (s + 1e-20f);
    }
    if (live) {
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
            if (j < k && j % L == r) {
                idx[t * k + j] = pe[j];
                w[t * k + j] = wt[j];
            }
    }
}

template <int L, int VPL, int KMAX>
hipError_t launch_l(const moe_config& c, const float* logits, int32_t* idx, float* w, hipStream_t s) {
    constexpr int tokens_per_block = (256 / kWave) * (kWave / L);
    const dim3 grid((unsigned)((c.T + tokens_per_block - 1) / tokens_per_block)), block(256);
    route_kernel<L, VPL, KMAX><<<grid, block, 0, s>>>(logits, c.T, c.E, c.k, c.score, c.renorm, idx, w);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const moe_config& c, const float* logits, int32_t* idx, float* w, hipStream_t s) {
    if (c.T == 0) return hipSuccess;
    if (c.k > 8) return launch_l<32, 32, kMaxTopK>(c, logits, idx, w, s);  // E <= 1024
    if (c.E <= 8) return launch_l<1, 8, 8>(c, logits, idx, w, s);
    if (c.E <= 16) return launch_l<1, 16, 8>(c, logits, idx, w, s);
    if (c.E <= 32) return launch_l<1, 32, 8>(c, logits, idx, w, s);
    if (c.E <= 64) return launch_l<2, 32, 8>(c, logits, idx, w, s);
    if (c.E <= 128) return launch_l<4, 32, 8>(c, logits, idx, w, s);
    if (c.E <= 256) return launch_l<8, 32, 8>(c, logits, idx, w, s);
    if (c.E <= 512) return launch_l<16, 32, 8>(c, logits, idx, w, s);
    return launch_l<32, 32, 8>(c, logits, idx, w, s);
}

}  // namespace moe
