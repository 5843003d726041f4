// gma_forward_noalloc: gma_forward for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Its scratch is one
// file-scope device array of GMA_NOALLOC_SCRATCH_BYTES; each GPU the library runs on holds its
// own copy at its own address until the process ends.
//
// In host code the array's name is only a host-side stand-in, never a device address: the
// device address is looked up once per device with hipGetSymbolAddress (with that device
// current) and kept in a per-device table, and only that address is handed to the kernels.
//
// Every call on one GPU shares that GPU's array.  No forward kernel relies on the scratch
// starting at zero (each writes every scratch byte it later reads within the same call), so
// nothing is cleared between calls; calls that overlap on one GPU (different streams, or
// different host threads without ordering) race on the array and must not be issued.
#include <mutex>

#include "gma_internal.h"

namespace {

__device__ __align__(256) unsigned char scratch[GMA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_ptr[kMaxDevices] = {};

// Device address of this device's scratch array; looked up on the first call per device.
void* scratch_address(void* stream, int* status) {
    int dev = -1;
    hipError_t e = stream ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) : hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *status = e != hipSuccess ? GMA_ERR_HIP : GMA_ERR_UNSUPPORTED;
        return nullptr;
    }
    std::lock_guard<std::mutex> guard(g_lock);
    if (!g_ptr[dev]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) {
            *status = GMA_ERR_HIP;
            return nullptr;
        }
        if (cur != dev && hipSetDevice(dev) != hipSuccess) {
            *status = GMA_ERR_HIP;
            return nullptr;
        }
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || !p) {
            *status = GMA_ERR_HIP;
            return nullptr;
        }
        g_ptr[dev] = p;
    }
    return g_ptr[dev];
}

}  // namespace

extern "C" int gma_forward_noalloc(const void* qr, const void* kr, const void* v, const float* mu,
                                   const float* var_raw, const float* prior_logits, int causal, float eps,
                                   void* out, float* gamma_out, const gma_desc* desc, void* stream) {
    const gma::ScratchSource src{GMA_NOALLOC_SCRATCH_BYTES, scratch_address};
    return gma::forward_with_scratch(qr, kr, v, mu, var_raw, prior_logits, causal, eps, out, gamma_out, desc,
                                     stream, src);
}
