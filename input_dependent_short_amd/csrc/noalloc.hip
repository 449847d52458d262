// noalloc.hip -- the device scratch of the allocation-free low-rank backward
// (dsc_lowrank_bwd_noalloc).  The bf16 backward adds its dz partial sums into
// an fp32 (B*T, R) accumulator before rounding them to bf16; callers that
// cannot allocate device memory (code under stream capture, serving loops,
// harnesses that forbid allocation) get that accumulator from this
// file-scope array instead of a workspace argument.
//
// Each device that runs the library holds its own copy of the array until
// the process ends.  Host code never passes the array's name to a kernel: in
// host code it is a host-side stand-in, not a device address.  The device
// address is taken once per device with hipGetSymbolAddress, with that
// device current, and kept.  Every call on one device shares its array, so
// calls that overlap in time on one device race (the backward clears the
// part it uses with a kernel before each use).
#include <hip/hip_runtime.h>

#include <mutex>

#include "dsc_kernels.h"

namespace dsc {
namespace {

static __device__ __align__(256) float scratch[kNoallocScratchFloats];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
float *g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(float **out) {
    *out = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_ptr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_ptr[dev] = static_cast<float *>(p);
    }
    *out = g_ptr[dev];
    return hipSuccess;
}

}  // namespace dsc
