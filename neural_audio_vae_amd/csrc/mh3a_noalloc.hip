// The static device scratch of mh3a_decode_noalloc: a file-scope device
// array that every GPU the library runs on holds until the process ends,
// so that a decode can run with no allocation at all (callers under HIP
// graph capture, serving loops, harnesses that forbid hipMalloc).
//
// In host code `scratch` names a host-side stand-in, not device memory:
// its device address on each GPU comes from hipGetSymbolAddress, looked up
// once per device with that device current, and only that address is ever
// handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "mh3a_internal.h"

namespace mh3a {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch_lookup(int device) {
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_ptr[device]) return hipSuccess;
    int prev = 0;
    hipError_t e = hipGetDevice(&prev);
    if (e != hipSuccess) return e;
    if (prev != device && (e = hipSetDevice(device)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (prev != device) {
        const hipError_t e2 = hipSetDevice(prev);
        if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[device] = p;
    return hipSuccess;
}

void* noalloc_scratch(int device) {
    if (device < 0 || device >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_mu);
    return g_ptr[device];
}

}  // namespace mh3a
