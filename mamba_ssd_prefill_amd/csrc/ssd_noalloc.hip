// ssd_noalloc.hip -- ssd_prefill_noalloc: ssd_prefill with the library's own static scratch as
// its workspace, for callers that cannot allocate (declared in include/mamba_ssd.h).
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/mamba_ssd.h"
#include "ssd_api_internal.h"

#define SSD_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

// The workspace of ssd_prefill_noalloc: one copy per GPU, at its own device address.  Host code
// never uses this name as an address (it is a host-side stand-in); it uses scratch_ptr().
static __device__ __align__(256) unsigned char scratch[SSD_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// The current device's address of `scratch`, looked up once per device with that device
// current (hipGetSymbolAddress); nullptr when the lookup fails.
void* scratch_ptr(hipError_t* err) {
    static std::mutex mu;
    static void* ptr[kMaxDevices] = {};
    int dev = 0;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!ptr[dev]) {
        void* p = nullptr;
        *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (*err != hipSuccess) return nullptr;
        ptr[dev] = p;
    }
    return ptr[dev];
}

}  // namespace

SSD_EXPORT ssd_status_t ssd_prefill_noalloc(const ssd_params_t* p, const void* x, const void* dt, const float* A,
                                           const void* B, const void* C, const float* D, const float* dt_bias,
                                           const void* initial_state, void* y, void* final_state, void* stream) {
    const ssd_status_t s = ssd_validate(p);
    if (s != SSD_OK) return s;
    if (ssd_prefill_workspace_size(p) > SSD_NOALLOC_SCRATCH_BYTES) return SSD_ERR_SCRATCH_TOO_SMALL;
    hipError_t e = hipSuccess;
    void* ws = scratch_ptr(&e);
    if (!ws) return SSD_ERR_HIP;
    return ssd::prefill_impl(p, x, dt, A, B, C, D, dt_bias, initial_state, y, final_state, ws,
                             SSD_NOALLOC_SCRATCH_BYTES, stream, nullptr, nullptr, nullptr);
}
