// Library-owned device scratch for the allocation-free prefill entry point
// (rb_matmul_noalloc): the workspace of the Route B prefill's activation
// pre-pass, as a file-scope device array instead of caller memory.
//
// Each GPU the library runs on holds its own copy of `scratch` (kScratchBytes)
// until the process ends.  In host code the array's name is only a stand-in
// for the device symbol, so its device address is looked up once per device
// with hipGetSymbolAddress, with that device current, and the looked-up
// address is what kernels and copies are given.
#include <mutex>

#include "common.h"

namespace dmm {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];        // device address of `scratch`, per device

}  // namespace

hipError_t scratch_of_current_device(void** out) {
    int dev = -1;
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
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace dmm
