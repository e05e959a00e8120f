// Fixed device scratch of libkvq for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): kvq_decode_attention_noalloc takes its split workspace from here.
//
// Every GPU the library runs on holds its own copy of the array until the
// process ends. In host code `scratch` names a host-side stand-in, not a device
// address: the device address is taken once per device, with that device
// current, by hipGetSymbolAddress, and only that address is ever handed to
// kernels. Calls on one GPU share its array: calls that overlap on one GPU race.
// The decode workspace needs no clearing (every partial a kernel reads was
// written by the same call).
#include <hip/hip_runtime.h>

#include <mutex>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace kvq
