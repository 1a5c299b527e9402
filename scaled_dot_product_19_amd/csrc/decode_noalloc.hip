// decode_noalloc.hip -- the library-owned split workspace of
// sdpa_decode_paged_noalloc (include/sdpa.h), for callers that cannot
// allocate device memory around a call: code under stream capture, tight
// serving loops, harnesses that forbid hipMalloc.
//
// The workspace is one file-scope __device__ array, `scratch`, of
// kDecodeScratchBytes per GPU; every GPU the library runs on holds its own
// copy from the time the code object is loaded until the process ends.  In
// host code `scratch` names a host-side stand-in, not a device address, so
// its device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and kept; kernels only ever receive that address.
// All calls on one GPU share its array and it keeps the last call's
// contents: the split kernels write every partial the combine reads, so
// nothing needs clearing, but calls that overlap on one GPU race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "sdpa_launch.h"

namespace sdpa {
namespace {

__device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once looked up

}  // namespace

hipError_t decode_scratch(void** ptr) {
    *ptr = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace sdpa
