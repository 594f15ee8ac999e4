// moe_forward without a caller workspace, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).
//
// The scratch space moe_forward takes from its workspace argument (the
// grouping's per-chunk counts, the grouped GEMMs' work-queue counters and
// K-split partial sums, the per-row routing weights) comes from `scratch`, a
// file-scope device array of kNoAllocScratchBytes that every device the
// library is loaded on holds until the process ends.  Its address on the
// current device is looked up once per device (hipGetSymbolAddress, with that
// device current, on the first call there) and kept; host code never uses the
// array's name as an address.  Nothing in it has to start at zero: the
// kernels that read it (counters included) write it first in the same call.
// Every call on one device shares that device's array, so calls that overlap
// on one device (different streams, or host threads without ordering) race.
#include <mutex>

#include "moe_internal.h"

namespace {

constexpr size_t kNoAllocScratchBytes = (size_t)68 << 20;  // 68 MiB
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices];  // the array's device address, per device

moe_status scratch_on_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return moe::set_error(MOE_ERR_HIP, "moe_forward_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return moe::set_error(MOE_ERR_UNSUPPORTED, "moe_forward_noalloc: device %d beyond the %d supported", dev,
                              kMaxDevices);
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return moe::set_error(MOE_ERR_HIP, "moe_forward_noalloc: hipGetSymbolAddress of the scratch array: %s",
                                  hipGetErrorString(e));
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_forward_noalloc(const moe_config* cfg, const float* logits, const float* bias,
                                          const void* x, const uint8_t* x_scale, const void* w1, const uint8_t* w1_scale,
                                          const void* w2, const uint8_t* w2_scale, void* y, int32_t* idx, float* w,
                                          int32_t* counts, int32_t* offsets, int32_t* row_map, int32_t* src_map,
                                          void* xp, uint8_t* xp_scale, void* h, uint8_t* h_scale, void* yp,
                                          void* gu_stash, int32_t* err, void* stream) {
    // a bad config: moe_forward reports it (with no workspace, before any device call)
    if (moe_rows_capacity(cfg) < 0)
        return moe_forward(cfg, logits, bias, x, x_scale, w1, w1_scale, w2, w2_scale, y, idx, w, counts, offsets,
                           row_map, src_map, xp, xp_scale, h, h_scale, yp, gu_stash, err, nullptr, 0, stream);
    const size_t need = moe_workspace_size(cfg);
    if (need > kNoAllocScratchBytes)
        return moe::set_error(MOE_ERR_WORKSPACE,
                              "moe_forward_noalloc: this config needs %zu bytes of scratch, above the %zu of the "
                              "library's static array (use moe_forward with a workspace)",
                              need, kNoAllocScratchBytes);
    void* ws = nullptr;
    moe_status st = scratch_on_current_device(&ws);
    if (st) return st;
    return moe_forward(cfg, logits, bias, x, x_scale, w1, w1_scale, w2, w2_scale, y, idx, w, counts, offsets,
                       row_map, src_map, xp, xp_scale, h, h_scale, yp, gu_stash, err, ws, kNoAllocScratchBytes, stream);
}
