// Device scratch of the decode entry point that allocates nothing.
//
// For callers that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc): the decode's partial softmax states
// live in one file-scope device array instead of a caller workspace.  Every GPU the
// library runs on holds its own copy of the array until the process ends; its device
// address is looked up once per device, with that device current, and kept.  In host
// code the array's name is only a stand-in: kernels and copies get the looked-up address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"
#include "octopus_dag.h"

static __device__ __align__(256) unsigned char scratch[OCTOPUS_DECODE_SCRATCH_BYTES];

namespace octo {

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t decode_scratch(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace octo
