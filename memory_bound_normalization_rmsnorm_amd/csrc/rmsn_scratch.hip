// rmsn_scratch.hip -- the static device workspace of rmsnorm_bwd_noalloc.
//
// `scratch` holds the backward's fp32 dW partial rows for callers that cannot
// allocate device memory (code under HIP graph capture, serving loops that
// forbid hipMalloc). It lives in this file's code object: each GPU the
// library runs on holds its own copy, RMSN_NOALLOC_SCRATCH_BYTES long, until
// the process ends. In host code the name `scratch` is a host-side stand-in,
// not a device address; the device address of the current device's copy is
// looked up once per device with hipGetSymbolAddress and kept, and only that
// address is ever passed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>
#include <unordered_map>

#include "../../include/rmsnorm.h"
#include "rmsn_tables.h"

static __device__ __align__(256) float scratch[RMSN_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace rmsn {

namespace {
std::mutex g_scratch_mu;
std::unordered_map<int, void *> g_scratch;  // device ordinal -> that device's copy of `scratch`
}  // namespace

int scratch_region(int dev, void **ptr) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    auto it = g_scratch.find(dev);
    if (it != g_scratch.end()) {
        *ptr = it->second;
        return RMSN_OK;
    }
    // `dev` is the current device (the caller read it with hipGetDevice), so
    // this resolves that device's copy.
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return RMSN_EHIP;
    if ((reinterpret_cast<uintptr_t>(p) & 255u) != 0) return RMSN_EHIP;
    g_scratch.emplace(dev, p);
    *ptr = p;
    return RMSN_OK;
}

}  // namespace rmsn
