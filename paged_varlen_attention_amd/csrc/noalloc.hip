// noalloc.hip -- the device scratch behind pa_varlen_attention_noalloc: the
// split-KV partials (normalised partial outputs, log2 max and exp-sum of every
// (token, head, partition)) live in one file-scope device array instead of
// caller-allocated buffers, for callers that cannot allocate device memory.
//
// Each GPU the library runs on holds its own copy of the array until the
// process ends.  In host code the array's name is only a host-side stand-in,
// so its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/pa.h"
#include "pa_internal.h"

namespace pa {
namespace {

static __device__ __align__(256) char scratch[PA_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void *g_ptr[MAX_DEVICES] = {};

}  // namespace

hipError_t noalloc_scratch(void **ptr) {
    *ptr = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_ptr[dev] = p;
    }
    *ptr = g_ptr[dev];
    return hipSuccess;
}

}  // namespace pa
