// Routing backward: the gradient of the top-k weights and of the router
// logits, one wavefront per token.
//
// The forward (route.hip) gives route (t, j) the weight w[t][j] of its expert
// idx[t][j]: the softmax over all E logits p, p renormalised over the k
// chosen, or the sigmoid of the chosen logits normalised over the k chosen
// (the router of the TransformerEngine page "[JAX] Expert Parallelism: JAX
// primitives + VJPs", commit messages on the router); the combine forms
// y[t] = sum_j w[t][j] Yp[row_map[t][j]] (cudnn-frontend page "Add MoE +
// expert-parallel Python API surface, PyTorch reference, and tests",
// Summary).  For an upstream gradient dY of y:
//   dw[t][j]      = <dY[t], Yp[row_map[t][j]]>   (float32; 0 for a dropped route)
//   dlogits[t][e] = sum_j dw[t][j] * d w[t][j] / d logits[t][e]
// by the chain rule through that normalisation (the top-k choice itself is
// piecewise constant):
//   softmax:              dl_e = p_e (dw_e - sum_j dw_j p_j), over all E
//                         (dw_e = the dw of the route that chose e, else 0)
//   renormalised softmax: dl_c = w_c (dw_c - sum_j dw_j w_j) for the chosen
//                         c, 0 elsewhere (w is the softmax of the chosen logits)
//   normalised sigmoid:   dl_c = s_c (1 - s_c) (dw_c - sum_j dw_j w_j) / sum_j s_j
//                         for the chosen c, 0 elsewhere
// The normalising sum S carries the forward's + 1e-20 here too: when every
// chosen sigmoid underflows to 0 (chosen logits below about -88), S is 0, the
// forward's weights are 0, and so are these gradients (without the 1e-20 they
// would be 0/0).
//
// Lane layout as in route.hip: lane l holds the logits of experts l + 64 i.
// The dot products stream the token's dY row and its k Yp rows in 16-byte
// pieces, four routes at a time (their loads in flight together), and reduce
// across the wavefront; lane j then holds route j's dw, expert and weight.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kTokensPerBlock = 4;  // 4 wavefronts of 64 lanes
constexpr int kRoutesAtOnce = 4;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

// float32 values of 16 bytes of a row: 8 bf16 or 4 float
template <typename T_>
__device__ __forceinline__ void unpack16(const uint4& q, float (&v)[16 / sizeof(T_)]) {
    if constexpr (sizeof(T_) == 2) {
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    } else {
        v[0] = __uint_as_float(q.x);
        v[1] = __uint_as_float(q.y);
        v[2] = __uint_as_float(q.z);
        v[3] = __uint_as_float(q.w);
    }
}

template <typename T_, int EPL>
__global__ __launch_bounds__(256) void route_bwd_kernel(const T_* __restrict__ dy, const T_* __restrict__ yp,
                                                        const float* __restrict__ logits,
                                                        const int32_t* __restrict__ idx,
                                                        const int32_t* __restrict__ row_map, int T, int E, int k,
                                                        int H, int rows, int score, int renorm, float* __restrict__ dw_out,
                                                        float* __restrict__ dlogits) {
    constexpr int EL = 16 / sizeof(T_);  // elements per 16-byte piece
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * kTokensPerBlock + (threadIdx.x >> 6);
    if (t >= T) return;  // uniform per wavefront
    const int nch = H / EL;
    const uint4* const dyr = (const uint4*)(dy + (size_t)t * H);

    // dw of route j ends up in lane j
    float my_dw = 0.f;
    for (int j0 = 0; j0 < k; j0 += kRoutesAtOnce) {
        const uint4* yr[kRoutesAtOnce];
        bool live[kRoutesAtOnce];
#pragma unroll
        for (int u = 0; u < kRoutesAtOnce; ++u) {
            const int j = j0 + u;
            const int row = j < k ? row_map[(size_t)t * k + j] : -1;
            live[u] = row >= 0 && row < rows;  // rows outside Yp only for a bad row_map
            yr[u] = (const uint4*)(yp + (size_t)(live[u] ? row : 0) * H);
        }
        float acc[kRoutesAtOnce] = {};
        for (int c = lane; c < nch; c += kWave) {
            float d[EL];
            unpack16<T_>(dyr[c], d);
            uint4 q[kRoutesAtOnce];
#pragma unroll
            for (int u = 0; u < kRoutesAtOnce; ++u)
                if (live[u]) {  // each Yp row is read once: nontemporal
                    const u32x4 r = __builtin_nontemporal_load((const u32x4*)(yr[u] + c));
                    q[u] = make_uint4(r.x, r.y, r.z, r.w);
                }
#pragma unroll
            for (int u = 0; u < kRoutesAtOnce; ++u) {
                if (!live[u]) continue;
                float v[EL];
                unpack16<T_>(q[u], v);
#pragma unroll
                for (int i = 0; i < EL; ++i) acc[u] = fmaf(d[i], v[i], acc[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < kRoutesAtOnce; ++u) {
            const float s = wave_sum(acc[u]);
            if (lane == j0 + u) my_dw = live[u] ? s : 0.f;
        }
    }

    // lane j < k: route j's expert and forward score
    const bool mine = lane < k;
    const int my_e = mine ? idx[(size_t)t * k + lane] : -1;
    const bool my_ok = my_e >= 0 && my_e < E;
    const float my_l = my_ok ? logits[(size_t)t * E + my_e] : 0.f;
    float* const out = dlogits + (size_t)t * E;
    if (score == 0 && !renorm) {
        // softmax over all E: p needs every logit
        const float* const row = logits + (size_t)t * E;
        float v[EPL];
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane + kWave * i;
            v[i] = e < E ? row[e] : -INFINITY;
            m = fmaxf(m, v[i]);
        }
        m = wave_max(m);
        float z = 0.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            v[i] = __expf(v[i] - m);  // exp(-inf) = 0 past E
            z += v[i];
        }
        const float rz = 1.0f / wave_sum(z);
        const float my_p = my_ok ? __expf(my_l - m) * rz : 0.f;
        const float A = wave_sum(my_ok ? my_dw * my_p : 0.f);
        float ds[EPL] = {};
        for (int j = 0; j < k; ++j) {
            const int ej = __shfl(my_e, j, kWave);
            const float dj = __shfl(my_dw, j, kWave);
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                if (lane + kWave * i == ej) ds[i] += dj;
        }
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane + kWave * i;
            if (e < E) out[e] = v[i] * rz * (ds[i] - A);
        }
    } else {
        float a, S;
        if (score == 0) {  // renormalised softmax: the softmax of the chosen logits
            const float m = wave_max(my_ok ? my_l : -INFINITY);
            a = my_ok ? __expf(my_l - m) : 0.f;
        } else {  // normalised sigmoid
            a = my_ok ? 1.0f / (1.0f + __expf(-my_l)) : 0.f;
        }
        S = wave_sum(a) + 1e-20f;
        const float my_w = a / S;
        const float B = wave_sum(my_dw * my_w);
        // gradient of route j's logit
        const float my_g = score == 0 ? my_w * (my_dw - B) : a * (1.0f - a) * (my_dw - B) / S;
        float g[EPL] = {};
        for (int j = 0; j < k; ++j) {
            const int ej = __shfl(my_e, j, kWave);
            const float gj = __shfl(my_g, j, kWave);
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                if (lane + kWave * i == ej) g[i] += gj;
        }
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane + kWave * i;
            if (e < E) out[e] = g[i];
        }
    }
    if (dw_out && mine) dw_out[(size_t)t * k + lane] = my_dw;
}

template <typename T_>
hipError_t launch_t(const moe_config& c, const void* dy, const void* yp, const float* logits, const int32_t* idx,
                    const int32_t* row_map, float* dw, float* dlogits, hipStream_t s) {
    const dim3 grid((unsigned)((c.T + kTokensPerBlock - 1) / kTokensPerBlock)), block(256);
    const T_* d = (const T_*)dy;
    const T_* y = (const T_*)yp;
    const int sc = c.score == MOE_SIGMOID ? 1 : 0;
    const int rows = (int)((int64_t)c.T * c.k + (int64_t)c.E * (c.align - 1));  // R_cap
#define RB_LAUNCH(EPL)                                                                                   \
    route_bwd_kernel<T_, EPL><<<grid, block, 0, s>>>(d, y, logits, idx, row_map, c.T, c.E, c.k, c.H, rows, sc,       \
                                                     c.renorm, dw, dlogits)
    if (c.E <= 64) RB_LAUNCH(1);
    else if (c.E <= 128) RB_LAUNCH(2);
    else if (c.E <= 256) RB_LAUNCH(4);
    else if (c.E <= 512) RB_LAUNCH(8);
    else RB_LAUNCH(16);
#undef RB_LAUNCH
    return hipGetLastError();
}

}  // namespace

hipError_t launch_route_bwd(const moe_config& c, const void* dy, const void* yp, const float* logits,
                            const int32_t* idx, const int32_t* row_map, float* dw, float* dlogits, hipStream_t s) {
    if (c.T == 0) return hipSuccess;
    if (c.dtype == MOE_F32) return launch_t<float>(c, dy, yp, logits, idx, row_map, dw, dlogits, s);
    return launch_t<uint16_t>(c, dy, yp, logits, idx, row_map, dw, dlogits, s);
}

}  // namespace moe
