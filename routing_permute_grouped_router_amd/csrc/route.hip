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
//
// The per-lane scan of a pick is branch-free (compares and selects, two
// independent chains over the two halves of the lane's slots, so the
// dependent compare-select latency is halved), and the lane exchanges inside
// a row of 16 are DPP moves: quad permutes for partners 1 and 2 apart, then
// the half-row and row mirrors (lane i with 7 - i, 15 - i), which pair whole
// quads and half-rows once those agree.  Only groups of 32 lanes (E > 512)
// exchange through ds_bpermute.
//
// With an expert bias (TransformerEngine page, router commits: an optional
// expert routing bias with a zero bias matching no bias), the selection runs
// on the key fl32(logit + bias[e]) and each pick carries its unbiased logit
// along, from which the weights are formed exactly as without a bias.
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

// The value of the partner lane at stage OFF of a group reduction (stages
// run OFF = 1, 2, 4, ... so each stage pairs lanes whose earlier stages agree).
template <int OFF>
__device__ __forceinline__ int partner(int x) {
    if constexpr (OFF == 1) return __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);   // quad [1,0,3,2]
    else if constexpr (OFF == 2) return __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);  // quad [2,3,0,1]
    else if constexpr (OFF == 4) return __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false); // half-row mirror
    else if constexpr (OFF == 8) return __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false); // row mirror
    else return __shfl_xor(x, OFF, kWave);
}
template <int OFF>
__device__ __forceinline__ float partner(float x) {
    return __int_as_float(partner<OFF>(__float_as_int(x)));
}

// f(integral_constant<OFF>) for OFF = 1, 2, 4, ... < L
template <int L, class F>
__device__ __forceinline__ void for_stages(F&& f) {
    if constexpr (L > 1) f(std::integral_constant<int, 1>{});
    if constexpr (L > 2) f(std::integral_constant<int, 2>{});
    if constexpr (L > 4) f(std::integral_constant<int, 4>{});
    if constexpr (L > 8) f(std::integral_constant<int, 8>{});
    if constexpr (L > 16) f(std::integral_constant<int, 16>{});
}

template <int L, int VPL, int KMAX, bool BIAS>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits,
                                                    const float* __restrict__ bias, int T, int E, int k,
                                                    int score, int renorm, int32_t* __restrict__ idx,
                                                    float* __restrict__ w) {
    constexpr int TPW = kWave / L;  // tokens per wavefront
    const int lane = threadIdx.x & 63;
    const int r = lane % L;
    const int64_t t = ((int64_t)blockIdx.x * (256 / kWave) + (threadIdx.x >> 6)) * TPW + lane / L;
    const bool live = t < T;
    const float* row = logits + (live ? t : 0) * (int64_t)E;

    float v[VPL];   // logits
    float kv[VPL];  // selection keys: the logits, or fl32(logit + bias)
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
            if (BIAS) {
                const float4 b = ok ? *(const float4*)(bias + e) : make_float4(0.f, 0.f, 0.f, 0.f);
                kv[i] = q.x + b.x;
                kv[i + 1] = q.y + b.y;
                kv[i + 2] = q.z + b.z;
                kv[i + 3] = q.w + b.w;
            }
            avail |= ok ? 0xfu << i : 0u;
        }
    } else {
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int e = r * VPL + i;
            const bool ok = live && e < E;
            v[i] = ok ? row[e] : -INFINITY;
            if (BIAS) kv[i] = v[i] + (ok ? bias[e] : 0.f);
            avail |= ok ? 1u << i : 0u;
        }
    }
    if (!BIAS) {
#pragma unroll
        for (int i = 0; i < VPL; ++i) kv[i] = v[i];
    }
    // group-wide reductions (the L lanes of a group are consecutive and
    // aligned, so every partner stays inside it; a + b == b + a, so all lanes
    // of the group end with the same bits)
    auto gmax = [&](float x) {
        for_stages<L>([&](auto o) { x = fmaxf(x, partner<decltype(o)::value>(x)); });
        return x;
    };
    auto gsum = [&](float x) {
        for_stages<L>([&](auto o) { x += partner<decltype(o)::value>(x); });
        return x;
    };

    float pv[KMAX];  // the picks' unbiased logits
    int pe[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        pv[j] = -INFINITY;
        pe[j] = -1;
        if (j >= k) continue;
        // the lane's best available slot: slots in ascending order, a strictly
        // larger key replaces, so equal keys keep the lower slot; the first
        // available slot is always taken (a key of -inf included)
        constexpr int H2 = VPL / 2;
        float k0 = -INFINITY, k1 = -INFINITY, u0 = -INFINITY, u1 = -INFINITY;
        int i0 = -1, i1 = -1;
#pragma unroll
        for (int i = 0; i < H2; ++i) {
            const bool t0 = ((avail >> i) & 1u) & ((kv[i] > k0) | (i0 < 0));
            const bool t1 = ((avail >> (i + H2)) & 1u) & ((kv[i + H2] > k1) | (i1 < 0));
            k0 = t0 ? kv[i] : k0;
            i0 = t0 ? i : i0;
            k1 = t1 ? kv[i + H2] : k1;
            i1 = t1 ? i + H2 : i1;
            if constexpr (BIAS) {
                u0 = t0 ? v[i] : u0;
                u1 = t1 ? v[i + H2] : u1;
            }
        }
        const bool hi = (i1 >= 0) & ((k1 > k0) | (i0 < 0));  // ties keep the lower half
        float bk = hi ? k1 : k0;
        float bu = BIAS ? (hi ? u1 : u0) : bk;
        const int bi = hi ? i1 : i0;
        int be = bi < 0 ? 0x7fffffff : r * VPL + bi;  // no slot left: loses every comparison
        for_stages<L>([&](auto o) {
            constexpr int OFF = decltype(o)::value;
            // every lane reads its partner before any select: a DPP read
            // under a partial exec mask would see inactive lanes
            const float ok = partner<OFF>(bk);
            const int oe = partner<OFF>(be);
            const float ou = BIAS ? partner<OFF>(bu) : ok;
            const bool t = (ok > bk) | ((ok == bk) & (oe < be));
            bu = t ? ou : bu;
            bk = t ? ok : bk;
            be = t ? oe : be;
        });
        avail &= (be / VPL == r) ? ~(1u << (be % VPL)) : ~0u;  // the owning lane retires the pick
        pv[j] = BIAS ? bu : bk;
        pe[j] = be;
    }

    float wt[KMAX];
    if (score == MOE_SOFTMAX && !renorm) {
        // the first pick is the largest logit; with a bias it need not be
        float m = pv[0];
        if (BIAS) {
            m = -INFINITY;
#pragma unroll
            for (int i = 0; i < VPL; ++i)
                if (r * VPL + i < E) m = fmaxf(m, v[i]);
            m = gmax(m);
        }
        float z = 0.f;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            if (r * VPL + i < E) z += expf(v[i] - m);
        z = gsum(z);
#pragma unroll
        for (int j = 0; j < KMAX; ++j) wt[j] = j < k ? expf(pv[j] - m) / z : 0.f;
    } else if (score == MOE_SOFTMAX) {
        // p_j / (sum of the chosen p + 1e-20) with p the softmax over all E.
        // With m the largest chosen logit, a_j = exp(l_j - m) and
        // Zm = sum over all E of exp(l_e - m), this is a_j / (sum a + 1e-20 Zm)
        // (numerator and denominator times Z exp(max l - m)).  Without a bias
        // the chosen are the k largest logits, so sum a >= 1 and 1e-20 Zm <=
        // 1e-20 E < 2^-24: the term cannot change the float32 sum and only the
        // k chosen exponentials are formed.  A bias can choose experts whose p
        // is small enough for the 1e-20 to count, so then Zm is formed too
        // (a zero bias still gives the same bytes: the term rounds away).
        float m = pv[0];
        if (BIAS) {
#pragma unroll
            for (int j = 1; j < KMAX; ++j)
                if (j < k) m = fmaxf(m, pv[j]);
        }
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            wt[j] = j < k ? expf(pv[j] - m) : 0.f;
            s += wt[j];
        }
        if (BIAS) {
            float zm = 0.f;
#pragma unroll
            for (int i = 0; i < VPL; ++i)
                if (r * VPL + i < E) zm += expf(v[i] - m);
            s += 1e-20f * gsum(zm);
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
hipError_t launch_l(const moe_config& c, const float* logits, const float* bias, int32_t* idx, float* w,
                    hipStream_t s) {
    constexpr int tokens_per_block = (256 / kWave) * (kWave / L);
    const dim3 grid((unsigned)((c.T + tokens_per_block - 1) / tokens_per_block)), block(256);
    if (bias)
        route_kernel<L, VPL, KMAX, true><<<grid, block, 0, s>>>(logits, bias, c.T, c.E, c.k, c.score, c.renorm,
                                                                idx, w);
    else
        route_kernel<L, VPL, KMAX, false><<<grid, block, 0, s>>>(logits, nullptr, c.T, c.E, c.k, c.score,
                                                                 c.renorm, idx, w);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const moe_config& c, const float* logits, const float* bias, int32_t* idx, float* w,
                        hipStream_t s) {
    if (c.T == 0) return hipSuccess;
    if (c.k > 8) return launch_l<32, 32, kMaxTopK>(c, logits, bias, idx, w, s);  // E <= 1024
    if (c.E <= 8) return launch_l<1, 8, 8>(c, logits, bias, idx, w, s);
    if (c.E <= 16) return launch_l<1, 16, 8>(c, logits, bias, idx, w, s);
    if (c.E <= 32) return launch_l<1, 32, 8>(c, logits, bias, idx, w, s);
    if (c.E <= 64) return launch_l<2, 32, 8>(c, logits, bias, idx, w, s);
    if (c.E <= 128) return launch_l<4, 32, 8>(c, logits, bias, idx, w, s);
    if (c.E <= 256) return launch_l<8, 32, 8>(c, logits, bias, idx, w, s);
    if (c.E <= 512) return launch_l<16, 32, 8>(c, logits, bias, idx, w, s);
    return launch_l<32, 32, 8>(c, logits, bias, idx, w, s);
}

}  // namespace moe
