// Static device scratch for fftconv_forward_noalloc: the workspace of the
// forward kernels (the wide kernel's row-claim counters, the multi-pass
// path's f16 channel chunk and its counters) for callers that cannot
// allocate device memory.  Every GPU the library runs on holds one copy of
// the array from the first call on it until the process ends; all calls on
// one GPU share it, so calls that overlap in time on one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fftconv_internal.h"

namespace fftconv {
namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;

// Only device code and hipGetSymbolAddress may name this array: in host
// code the name is a host-side stand-in, not a device address.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_lock;
void* g_ptr[kMaxDevices];

}  // namespace

hipError_t scratch_buffer(int device, void** ptr, size_t* bytes) {
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> hold(g_lock);
    if (!g_ptr[device]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_ptr[device] = p;
    }
    *ptr = g_ptr[device];
    *bytes = kScratchBytes;
    return hipSuccess;
}

}  // namespace fftconv
