// Allocation-free forward: gdn_fwd_noalloc is gdn_fwd with its workspace
// taken from a static device array instead of a caller buffer, for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid allocation).
//
// The array below lives in this library's code object, one copy per GPU,
// held until the process ends. Host code never uses its name as an address:
// the device address of each GPU's copy is looked up once per device with
// hipGetSymbolAddress (with that device current) on the first call there,
// and only that address is handed to the kernels. Every call on one GPU
// shares that GPU's copy, so calls that overlap in time on one GPU race;
// the forward writes every workspace byte it later reads, so no clearing is
// needed between calls.
#include <hip/hip_runtime.h>

#include <mutex>
#include <stdio.h>

#include "gdn.h"
#include "gdn_launch.hpp"

namespace {

static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEV = 64;
std::mutex g_lock;
void *g_ptr[MAX_DEV] = {};

// Device address of the current device's copy of `scratch` (looked up once).
gdn_status_t scratch_of_current(void *&out) {
    int dev = 0;
    char msg[160];
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= MAX_DEV) {
        snprintf(msg, sizeof msg, "gdn_fwd_noalloc: no usable current device (%s)", hipGetErrorString(e));
        return gdn::fail_detail(GDN_EHIP, msg);
    }
    std::lock_guard<std::mutex> hold(g_lock);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            snprintf(msg, sizeof msg, "gdn_fwd_noalloc: scratch address lookup failed (%s)", hipGetErrorString(e));
            return gdn::fail_detail(GDN_EHIP, msg);
        }
        g_ptr[dev] = p;
    }
    out = g_ptr[dev];
    return GDN_OK;
}

} // namespace

extern "C" gdn_status_t gdn_fwd_noalloc(const gdn_shape_t *s, const void *q, const void *k, const void *v,
                                        const float *g, const float *beta, const float *A_log, const float *D,
                                        const float *h0, void *o, float *hT, void *ctx, void *stream) {
    const size_t need = gdn_fwd_workspace_size(s);
    if (need > (size_t)GDN_NOALLOC_SCRATCH_BYTES) {
        char msg[200];
        snprintf(msg, sizeof msg,
                 "gdn_fwd_noalloc: this shape needs %zu bytes of scratch; the static scratch holds %zu "
                 "(use gdn_fwd with a workspace)",
                 need, (size_t)GDN_NOALLOC_SCRATCH_BYTES);
        return gdn::fail_detail(GDN_EWORKSPACE, msg);
    }
    // an invalid shape (need == 0) is reported by the forward's own checks
    return gdn::fwd_entry(s, q, k, v, g, beta, A_log, D, h0, o, hT, ctx, nullptr,
                          (size_t)GDN_NOALLOC_SCRATCH_BYTES, stream, true, scratch_of_current);
}
