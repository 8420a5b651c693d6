// rmsn_probe.hip -- HBM roofline probes: copy, pure write, 2-read-1-write,
// and a pure read (used as a cache flush that leaves no dirty lines).
// Each lane streams 16-byte vectors; with a grid smaller than the vector
// count, lanes stride by the whole grid so every access of one instruction
// is contiguous across the wavefront. Each probe is built with and without
// the non-temporal hint on its loads and on its stores (variant bits 0 and
// 1), so the measured roofline is the best the device reaches, not the best
// of one access flavour.
#include <hip/hip_runtime.h>

#include "../../include/rmsnorm.h"
#include "../../include/rmsnorm_probe.h"
#include "rmsn_device.h"

namespace {

using rmsn::u32x4;
constexpr int kWG = 256;

template <bool NT>
__device__ __forceinline__ u32x4 ld(const u32x4 *p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}
template <bool NT>
__device__ __forceinline__ void st(u32x4 *p, const u32x4 &v) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

template <bool NTL, bool NTS>
__global__ void __launch_bounds__(kWG) probe_copy(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * kWG + threadIdx.x; i < n; i += (int64_t)gridDim.x * kWG)
        st<NTS>(dst + i, ld<NTL>(src + i));
}

template <bool NTL, bool NTS>
__global__ void __launch_bounds__(kWG) probe_write(u32x4 *__restrict__ dst, int64_t n) {
    const u32x4 v = {0x3f800000u, 0x3f800000u, 0x3f800000u, 0x3f800000u};
    for (int64_t i = (int64_t)blockIdx.x * kWG + threadIdx.x; i < n; i += (int64_t)gridDim.x * kWG) st<NTS>(dst + i, v);
}

template <bool NTL, bool NTS>
__global__ void __launch_bounds__(kWG)
probe_add(const u32x4 *__restrict__ a, const u32x4 *__restrict__ b, u32x4 *__restrict__ c, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * kWG + threadIdx.x; i < n; i += (int64_t)gridDim.x * kWG)
        st<NTS>(c + i, ld<NTL>(a + i) + ld<NTL>(b + i));
}

// Reads every vector; the (practically never taken) data-dependent store keeps
// the loads alive without writing back anything.
template <bool NTL, bool NTS>
__global__ void __launch_bounds__(kWG) probe_read(const u32x4 *__restrict__ src, u32x4 *__restrict__ sink, int64_t n) {
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int64_t i = (int64_t)blockIdx.x * kWG + threadIdx.x; i < n; i += (int64_t)gridDim.x * kWG) acc ^= ld<NTL>(src + i);
    if (acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u && acc.z == 0x94d049bbu && acc.w == 0x2545f491u) st<NTS>(sink, acc);
}

bool bad(const void *p) { return !p || (reinterpret_cast<uintptr_t>(p) & 15u); }

int grid_for(size_t bytes, int64_t grid, int variant, int64_t *n, unsigned *g) {
    if (bytes % 16 || variant < 0 || variant > 3) return RMSN_EINVAL;
    *n = (int64_t)(bytes / 16);
    int64_t full = (*n + kWG - 1) / kWG;
    int64_t gg = grid > 0 && grid < full ? grid : full;
    if (gg > INT32_MAX) return RMSN_EINVAL;
    *g = (unsigned)gg;
    return RMSN_OK;
}

int done(hipError_t e) { return e == hipSuccess ? RMSN_OK : RMSN_EHIP; }

#define RMSN_PROBE_DISPATCH(K, VARIANT, ...)                      \
    switch (VARIANT) {                                            \
    case 0: hipLaunchKernelGGL((K<false, false>), __VA_ARGS__); break; \
    case 1: hipLaunchKernelGGL((K<true, false>), __VA_ARGS__); break;  \
    case 2: hipLaunchKernelGGL((K<false, true>), __VA_ARGS__); break;  \
    default: hipLaunchKernelGGL((K<true, true>), __VA_ARGS__); break;  \
    }

}  // namespace

extern "C" {

int rmsn_probe_copy(const void *src, void *dst, size_t bytes, int64_t grid, int variant, void *stream) {
    if (bad(src) || bad(dst)) return RMSN_EINVAL;
    int64_t n; unsigned g;
    int st = grid_for(bytes, grid, variant, &n, &g);
    if (st != RMSN_OK || n == 0) return st;
    RMSN_PROBE_DISPATCH(probe_copy, variant, dim3(g), dim3(kWG), 0, static_cast<hipStream_t>(stream),
                        static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), n)
    return done(hipGetLastError());
}

int rmsn_probe_write(void *dst, size_t bytes, int64_t grid, int variant, void *stream) {
    if (bad(dst)) return RMSN_EINVAL;
    int64_t n; unsigned g;
    int st = grid_for(bytes, grid, variant, &n, &g);
    if (st != RMSN_OK || n == 0) return st;
    RMSN_PROBE_DISPATCH(probe_write, variant, dim3(g), dim3(kWG), 0, static_cast<hipStream_t>(stream),
                        static_cast<u32x4 *>(dst), n)
    return done(hipGetLastError());
}

int rmsn_probe_read(const void *src, size_t bytes, int64_t grid, int variant, void *sink, void *stream) {
    if (bad(src) || bad(sink)) return RMSN_EINVAL;
    int64_t n; unsigned g;
    int st = grid_for(bytes, grid, variant, &n, &g);
    if (st != RMSN_OK || n == 0) return st;
    RMSN_PROBE_DISPATCH(probe_read, variant, dim3(g), dim3(kWG), 0, static_cast<hipStream_t>(stream),
                        static_cast<const u32x4 *>(src), static_cast<u32x4 *>(sink), n)
    return done(hipGetLastError());
}

int rmsn_probe_add(const void *a, const void *b, void *c, size_t bytes, int64_t grid, int variant, void *stream) {
    if (bad(a) || bad(b) || bad(c)) return RMSN_EINVAL;
    int64_t n; unsigned g;
    int st = grid_for(bytes, grid, variant, &n, &g);
    if (st != RMSN_OK || n == 0) return st;
    RMSN_PROBE_DISPATCH(probe_add, variant, dim3(g), dim3(kWG), 0, static_cast<hipStream_t>(stream),
                        static_cast<const u32x4 *>(a), static_cast<const u32x4 *>(b), static_cast<u32x4 *>(c), n)
    return done(hipGetLastError());
}

}  // extern "C"
