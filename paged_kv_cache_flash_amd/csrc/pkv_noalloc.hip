// pkv_noalloc.hip -- the device-resident scratch buffer of
// pkv_varlen_fwd_noalloc (callers that cannot allocate device memory).
//
// The split-KV partials of a forward normally live in a caller-owned
// workspace. Here they live in one file-scope device array instead, of
// kScratchBytes, which each GPU the library runs on holds until the process
// ends. In host code the array's name is a host-side stand-in, not a device
// address: its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pkv_kernels.h"

namespace {

static __device__ __align__(256) uint8_t scratch[pkv::kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

namespace pkv {

hipError_t scratch_for_current_device(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_ptr[dev] = p;
    }
    *ptr = g_ptr[dev];
    return hipSuccess;
}

}  // namespace pkv
