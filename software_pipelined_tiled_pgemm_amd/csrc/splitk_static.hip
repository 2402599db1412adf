// Static scratch buffer of the allocation-free split-K entry point
// (pgemm_f16_splitk_noalloc): the fp32 partial products live in a file-scope
// device array instead of a caller workspace.  The HIP runtime gives every
// device that loads this code object its own copy, held until the process
// ends.  In host code `scratch` is only a stand-in for the symbol, not a
// device address: its address on a device comes from hipGetSymbolAddress,
// looked up once per device with that device current, and only that
// pointer is passed to kernels.

#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/pgemm.h"
#include "internal.h"

static __device__ __align__(256) float scratch[PGEMM_STATIC_SCRATCH_BYTES / sizeof(float)];

namespace pgemm {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
float* g_scratch[kMaxDevices] = {};

}  // namespace

hipError_t static_scratch(float** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch[dev] = static_cast<float*>(p);
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace pgemm
