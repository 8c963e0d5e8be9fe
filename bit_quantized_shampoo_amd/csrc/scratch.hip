// Device scratch of the allocation-free entry point (shampoo4_gemm_batched_static): one
// file-scope device array per GPU holds the descriptor table and tile prefix of a batched
// product, so that callers that may not allocate device memory still pass only their
// operands.  Host code never uses the array's name as a device address: its address on
// each device is looked up once, with that device current, and kept.
#include <mutex>

#include "kernels.hpp"

namespace s4 {

namespace {

static __device__ __align__(256) uint8_t scratch[GEMM_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t gemm_static_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace s4
