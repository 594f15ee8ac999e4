// Routing: score function + top-k + normalisation, one wavefront per token.
//
// Follows the fp32 router with softmax / sigmoid scores and the
// "sum of selected + 1e-20" normalisation described on the TransformerEngine
// page "[JAX] Expert Parallelism: JAX primitives + VJPs" (commit messages on
// the router), and the routing step of the cudnn-frontend page "Add MoE +
// expert-parallel Python API surface, PyTorch reference, and tests" (Summary).
//
// Each lane holds EPL logits of its token (expert e = lane + 64*i).  The k
// selections are k wave-wide arg-max reductions over (logit desc, expert asc)
// among the experts not yet taken, so equal logits resolve to the lower expert
// index and slot j holds the j-th largest.  Lane j keeps the j-th pick, so the
// normalising sums are plain wave reductions over lanes < k.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kTokensPerBlock = 4;  // 4 wavefronts of 64 lanes

__device__ __forceinline__ bool better(float v, int e, float bv, int be) {
    return v > bv || (v == bv && e < be);
}

template <int EPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                    int score, int renorm, int32_t* __restrict__ idx,
                                                    float* __restrict__ w) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * kTokensPerBlock + (threadIdx.x >> 6);
    if (t >= T) return;  // uniform per wavefront
    const float* row = logits + (int64_t)t * E;

    float v[EPL];
    bool avail[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + kWave * i;
        avail[i] = e < E;
        v[i] = avail[i] ? row[e] : -INFINITY;
    }

    float my_v = -INFINITY;
    int my_e = -1;
    for (int j = 0; j < k; ++j) {
        float bv = -INFINITY;
        int be = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane + kWave * i;
            if (avail[i] && better(v[i], e, bv, be)) {
                bv = v[i];
                be = e;
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const float ov = __shfl_xor(bv, off, kWave);
            const int oe = __shfl_xor(be, off, kWave);
            if (better(ov, oe, bv, be)) {
                bv = ov;
                be = oe;
            }
        }
        if (lane == j) {
            my_v = bv;
            my_e = be;
        }
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (lane + kWave * i == be) avail[i] = false;
    }

    float wt;
    if (score == MOE_SOFTMAX) {
        const float m = __shfl(my_v, 0, kWave);  // the first pick is the maximum
        float z = 0.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (lane + kWave * i < E) z += expf(v[i] - m);
        z = wave_sum(z);
        const float p = lane < k ? expf(my_v - m) / z : 0.f;
        if (renorm) {
            const float s = wave_sum(p);
            wt = p / (s + 1e-20f);
        } else {
            wt = p;
        }
    } else {
        const float sg = lane < k ? 1.0f / (1.0f + expf(-my_v)) : 0.f;
        const float s = wave_sum(sg);
        wt = sg / (s + 1e-20f);
    }
    if (lane < k) {
        idx[(int64_t)t * k + lane] = my_e;
        w[(int64_t)t * k + lane] = wt;
    }
}

}  // namespace

hipError_t launch_route(const moe_config& c, const float* logits, int32_t* idx, float* w, hipStream_t s) {
    if (c.T == 0) return hipSuccess;
    const dim3 grid((c.T + kTokensPerBlock - 1) / kTokensPerBlock), block(256);
    const int epl = (c.E + kWave - 1) / kWave;
    if (epl <= 1)
        route_kernel<1><<<grid, block, 0, s>>>(logits, c.T, c.E, c.k, c.score, c.renorm, idx, w);
    else if (epl <= 2)
        route_kernel<2><<<grid, block, 0, s>>>(logits, c.T, c.E, c.k, c.score, c.renorm, idx, w);
    else if (epl <= 4)
        route_kernel<4><<<grid, block, 0, s>>>(logits, c.T, c.E, c.k, c.score, c.renorm, idx, w);
    else if (epl <= 8)
        route_kernel<8><<<grid, block, 0, s>>>(logits, c.T, c.E, c.k, c.score, c.renorm, idx, w);
    else
        route_kernel<16><<<grid, block, 0, s>>>(logits, c.T, c.E, c.k, c.score, c.renorm, idx, w);
    return hipGetLastError();
}

}  // namespace moe
