// Fixed device scratch for the entry point that allocates nothing
// (trsm_lln_noalloc): callers under HIP graph capture, serving loops that
// must not allocate, and harnesses that forbid hipMalloc.
//
// The blocked path's workspace (inverted diagonal blocks, the panel buffer,
// split-K partial sums) comes from this file-scope device array instead of
// hipMalloc.  Each GPU the library runs on holds its own copy of the array
// until the process ends.  In host code the array's name stands for a host
// stub, not a device address: the device address of each GPU's copy is taken
// once per device with hipGetSymbolAddress (with that device current) and
// only that address is handed to kernels.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>

#include "trsm.h"
#include "trsm_internal.h"

namespace trsm {
namespace {

static __device__ __align__(256) unsigned char scratch[TRSM_NOALLOC_MAX_WORKSPACE_BYTES];

std::mutex g_scratch_mu;
std::map<int, void *> g_scratch_ptr;  // device -> address of its copy of `scratch`

}  // namespace

hipError_t noalloc_scratch(int dev, void **out, size_t *bytes) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    auto it = g_scratch_ptr.find(dev);
    if (it == g_scratch_ptr.end()) {
        // `dev` is the current device (the caller took it from hipGetDevice)
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        it = g_scratch_ptr.emplace(dev, p).first;
    }
    *out = it->second;
    *bytes = sizeof(scratch);
    return hipSuccess;
}

}  // namespace trsm
