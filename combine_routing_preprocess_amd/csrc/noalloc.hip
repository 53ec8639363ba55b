// The grouped expert MLP for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): the FC1 -> FC2 activation scratch is a file-scope device array
// of fixed size instead of a caller-provided buffer.
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe_internal.h"

namespace {

// One copy per GPU the library runs on, held until the process ends.
__device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};   // device address of `scratch` per device

// Address of the current device's copy of `scratch`, looked up once per
// device (with that device current) and kept.  Host code never passes the
// array's name itself to a kernel or copy: on the host it is only a stand-in
// for the device symbol.
int scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_EHIP;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_EHIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return MOE_OK;
}

}  // namespace

extern "C" int moe_grouped_swiglu_mlp_noalloc(const moe_handle* h, int32_t F, int32_t wdtype, const void* d_perm,
                                              const float* d_perm_scales, const void* d_w1,
                                              const float* d_w1_scales, const void* d_w2,
                                              const float* d_w2_scales, void* d_expert_out, void* stream) {
    if (!h) return MOE_EINVAL;
    // every host check (and the size limit) before the first HIP call
    int rc = moe::check_mlp_host(h, F, wdtype, d_perm, d_perm_scales, d_w1, d_w1_scales, d_w2, d_w2_scales,
                                 d_expert_out);
    if (rc) return rc;
    if (moe_mlp_scratch_bytes(h, F, wdtype) > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ENOSPC;
    void* p = nullptr;
    rc = scratch_address(&p);
    if (rc) return rc;
    return moe_grouped_swiglu_mlp(h, F, wdtype, d_perm, d_perm_scales, d_w1, d_w1_scales, d_w2, d_w2_scales, p,
                                  (size_t)MOE_NOALLOC_SCRATCH_BYTES, d_expert_out, stream);
}
