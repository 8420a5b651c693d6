// rmsn_probe.hip -- HBM roofline probes: copy, pure write, 2-read-1-write.
// Each lane streams 16-byte vectors; with a grid smaller than the vector
// count, lanes stride by the whole grid so every access of one instruction
// is contiguous across the wavefront.
#include <hip/hip_runtime.h>

#include "../../include/rmsnorm.h"
#include "../../include/rmsnorm_probe.h"
#include "rmsn_device.h"

namespace {

using rmsn::u32x4;
constexpr int kWG = 256;

__global__ void __launch_bounds__(kWG) probe_copy(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * kWG + threadIdx.x; i < n; i += (int64_t)gridDim.x * kWG) dst[i] = src[i];
}

__global__ void __launch_bounds__(kWG) probe_write(u32x4 *__restrict__ dst, int64_t n) {
    const u32x4 v = {0x3f800000u, 0x3f800000u, 0x3f800000u, 0x3f800000u};
    for (int64_t i = (int64_t)blockIdx.x * kWG + threadIdx.x; i < n; i += (int64_t)gridDim.x * kWG) dst[i] = v;
}

__global__ void __launch_bounds__(kWG)
probe_add(const u32x4 *__restrict__ a, const u32x4 *__restrict__ b, u32x4 *__restrict__ c, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * kWG + threadIdx.x; i < n; i += (int64_t)gridDim.x * kWG) c[i] = a[i] + b[i];
}

bool bad(const void *p) { return !p || (reinterpret_cast<uintptr_t>(p) & 15u); }

int grid_for(size_t bytes, int64_t grid, int64_t *n, unsigned *g) {
    if (bytes % 16) return RMSN_EINVAL;
    *n = (int64_t)(bytes / 16);
    int64_t full = (*n + kWG - 1) / kWG;
    int64_t gg = grid > 0 && grid < full ? grid : full;
    if (gg > INT32_MAX) return RMSN_EINVAL;
    *g = (unsigned)gg;
    return RMSN_OK;
}

int done(hipError_t e) { return e == hipSuccess ? RMSN_OK : RMSN_EHIP; }

}  // namespace

extern "C" {

int rmsn_probe_copy(const void *src, void *dst, size_t bytes, int64_t grid, void *stream) {
    if (bad(src) || bad(dst)) return RMSN_EINVAL;
    int64_t n; unsigned g;
    int st = grid_for(bytes, grid, &n, &g);
    if (st != RMSN_OK || n == 0) return st;
    hipLaunchKernelGGL(probe_copy, dim3(g), dim3(kWG), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), n);
    return done(hipGetLastError());
}

int rmsn_probe_write(void *dst, size_t bytes, int64_t grid, void *stream) {
    if (bad(dst)) return RMSN_EINVAL;
    int64_t n; unsigned g;
    int st = grid_for(bytes, grid, &n, &g);
    if (st != RMSN_OK || n == 0) return st;
    hipLaunchKernelGGL(probe_write, dim3(g), dim3(kWG), 0, static_cast<hipStream_t>(stream),
                       static_cast<u32x4 *>(dst), n);
    return done(hipGetLastError());
}

int rmsn_probe_add(const void *a, const void *b, void *c, size_t bytes, int64_t grid, void *stream) {
    if (bad(a) || bad(b) || bad(c)) return RMSN_EINVAL;
    int64_t n; unsigned g;
    int st = grid_for(bytes, grid, &n, &g);
    if (st != RMSN_OK || n == 0) return st;
    hipLaunchKernelGGL(probe_add, dim3(g), dim3(kWG), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4 *>(a), static_cast<const u32x4 *>(b), static_cast<u32x4 *>(c), n);
    return done(hipGetLastError());
}

}  // extern "C"
