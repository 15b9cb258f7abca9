// scan_noalloc.hip -- the device scratch array of ssm_selective_scan_fwd_noalloc.
//
// That entry point runs the selective scan with its workspace (segment records
// and the carry between chained launches) in this fixed array instead of
// caller memory, for callers that cannot allocate device memory.  Each device
// the library runs on holds its own copy of the array for the life of the
// process.  In host code the array's name stands for a host-side shadow, not
// a device address: its device address is looked up with hipGetSymbolAddress,
// once per device with that device current, and only that address is ever
// passed on.
#include <mutex>

#include "ssm_internal.h"

namespace ssm {
namespace {

static_assert(SSM_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size must keep 256-byte alignment");

static __device__ __align__(256) char scratch[SSM_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of scratch per device, once looked up

}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, void **out) {
    *out = nullptr;
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    int dev = cur;
    if (stream != nullptr) {
        e = hipStreamGetDevice(stream, &dev);
        if (e != hipSuccess) return e;
    }
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t r = dev != cur ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess) return e;
        if (r != hipSuccess) return r;
        if (p == nullptr || reinterpret_cast<uintptr_t>(p) % 256 != 0) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace ssm
