// rmsn_baseline.hip -- unfused multi-kernel RMSNorm (the reference point for
// what fusion saves) and the separate rounding add.
//
// Same values as the fused kernels (per row: rstd = 1/sqrt(sum x^2 / N + eps),
// y = x rstd w; dx = r dy w - x r^3 S / N, S = sum dy w x; dW = sum_rows
// dy x r), with each step in a kernel of its own, so every kernel boundary
// sends the row through HBM again. Accesses are 16-byte vectors, coalesced
// across a wavefront; sums are fp32; dW is reduced without atomics in a fixed
// order.
#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>

#include "../../include/rmsnorm.h"
#include "../../include/rmsnorm_baseline.h"
#include "rmsn_device.h"

namespace rmsn_base {

using rmsn::Elem;
using rmsn::bf16_t;
using rmsn::f16_t;
using rmsn::u32x4;

constexpr int kWG = 256;
constexpr int kRowsPerWG = kWG / 64;  // one wavefront per row in the row kernels
constexpr int kPartialRows = 256;     // row chunks of the dW column kernel (at least, when M allows)
constexpr int kAlign = 64;            // partial-row stride in floats (256 bytes)
constexpr int64_t kMaxGrid = int64_t(1) << 22;

// the EPV weights paired with activation vector c of a row
template <typename T, typename TW>
__device__ __forceinline__ void load_w(const TW *__restrict__ w, int32_t c, float (&g)[Elem<T>::kPerVec]) {
    const u32x4 *wp = reinterpret_cast<const u32x4 *>(w);
    if constexpr (sizeof(TW) == sizeof(T)) {
        Elem<TW>::unpack(wp[c], g);
    } else {
        float a[4], b[4];
        Elem<float>::unpack(wp[2 * c], a);
        Elem<float>::unpack(wp[2 * c + 1], b);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            g[e] = a[e];
            g[4 + e] = b[e];
        }
    }
}

// ---- forward ----------------------------------------------------------------

template <typename T>
__global__ void __launch_bounds__(kWG)
un_rstd(const T *__restrict__ x, float eps, int64_t M, int32_t N, int32_t nvec, float *__restrict__ rstd) {
    const int lane = threadIdx.x & 63;
    const float n = (float)N;
    for (int64_t row = (int64_t)blockIdx.x * kRowsPerWG + (threadIdx.x >> 6); row < M;
         row += (int64_t)gridDim.x * kRowsPerWG) {
        const u32x4 *xr = reinterpret_cast<const u32x4 *>(x + row * N);
        float ss = 0.f;
        for (int32_t v = lane; v < nvec; v += 64) ss = Elem<T>::sumsq(xr[v], ss);
        ss = rmsn::group_sum<64>(ss);
        if (lane == 0) rstd[row] = __frsqrt_rn(ss / n + eps);
    }
}

template <typename T, typename TW>
__global__ void __launch_bounds__(kWG)
un_scale(const T *__restrict__ x, const TW *__restrict__ w, const float *__restrict__ rstd, T *__restrict__ y,
         int64_t total, int32_t nvec) {
    constexpr int EPV = Elem<T>::kPerVec;
    const u32x4 *xv = reinterpret_cast<const u32x4 *>(x);
    u32x4 *yv = reinterpret_cast<u32x4 *>(y);
    for (int64_t i = (int64_t)blockIdx.x * kWG + threadIdx.x; i < total; i += (int64_t)gridDim.x * kWG) {
        const int64_t row = i / nvec;
        const int32_t c = (int32_t)(i - row * nvec);
        const float r = rstd[row];
        float f[EPV], g[EPV];
        Elem<T>::unpack(xv[i], f);
        load_w<T, TW>(w, c, g);
#pragma unroll
        for (int k = 0; k < EPV; ++k) f[k] = (f[k] * r) * g[k];
        yv[i] = Elem<T>::pack(f);
    }
}

// ---- backward ---------------------------------------------------------------

template <typename T, typename TW>
__global__ void __launch_bounds__(kWG)
un_dot(const T *__restrict__ x, const TW *__restrict__ w, const T *__restrict__ dy, int64_t M, int32_t N,
       int32_t nvec, float *__restrict__ s) {
    constexpr int EPV = Elem<T>::kPerVec;
    const int lane = threadIdx.x & 63;
    for (int64_t row = (int64_t)blockIdx.x * kRowsPerWG + (threadIdx.x >> 6); row < M;
         row += (int64_t)gridDim.x * kRowsPerWG) {
        const u32x4 *xr = reinterpret_cast<const u32x4 *>(x + row * N);
        const u32x4 *gr = reinterpret_cast<const u32x4 *>(dy + row * N);
        float acc = 0.f;
        for (int32_t v = lane; v < nvec; v += 64) {
            float fx[EPV], fg[EPV], fw[EPV];
            Elem<T>::unpack(xr[v], fx);
            Elem<T>::unpack(gr[v], fg);
            load_w<T, TW>(w, v, fw);
#pragma unroll
            for (int k = 0; k < EPV; ++k) acc = __builtin_fmaf(fg[k] * fw[k], fx[k], acc);
        }
        acc = rmsn::group_sum<64>(acc);
        if (lane == 0) s[row] = acc;
    }
}

template <typename T, typename TW>
__global__ void __launch_bounds__(kWG)
un_dx(const T *__restrict__ x, const TW *__restrict__ w, const T *__restrict__ dy, const float *__restrict__ rstd,
      const float *__restrict__ s, T *__restrict__ dx, int64_t total, int32_t nvec, float n) {
    constexpr int EPV = Elem<T>::kPerVec;
    const u32x4 *xv = reinterpret_cast<const u32x4 *>(x);
    const u32x4 *gv = reinterpret_cast<const u32x4 *>(dy);
    u32x4 *ov = reinterpret_cast<u32x4 *>(dx);
    for (int64_t i = (int64_t)blockIdx.x * kWG + threadIdx.x; i < total; i += (int64_t)gridDim.x * kWG) {
        const int64_t row = i / nvec;
        const int32_t c = (int32_t)(i - row * nvec);
        const float r = rstd[row];
        const float cc = r * (r * (r * (s[row] / n)));
        float fx[EPV], fg[EPV], fw[EPV];
        Elem<T>::unpack(xv[i], fx);
        Elem<T>::unpack(gv[i], fg);
        load_w<T, TW>(w, c, fw);
#pragma unroll
        for (int k = 0; k < EPV; ++k) fx[k] = __builtin_fmaf(-fx[k], cc, r * (fg[k] * fw[k]));
        ov[i] = Elem<T>::pack(fx);
    }
}

// dW column partials. A workgroup covers `cols` consecutive activation vectors
// (cols = min(nvec, kWG)) for kWG / cols row chunks: lane t takes vector
// bx*cols + t % cols of chunk by*(kWG/cols) + t / cols, sums dy x rstd over
// the chunk's rows (rows chunk*rpc .. chunk*rpc+rpc-1, ascending) and writes
// partial[chunk][columns of that vector]. Narrow rows so still fill the
// workgroup.
template <typename T>
__global__ void __launch_bounds__(kWG)
un_dw_partial(const T *__restrict__ x, const T *__restrict__ dy, const float *__restrict__ rstd, int64_t M,
              int32_t N, int32_t nvec, int32_t cols, int64_t rpc, float *__restrict__ partial, int64_t ldp) {
    constexpr int EPV = Elem<T>::kPerVec;
    const int cpw = kWG / cols;
    if ((int)threadIdx.x >= cols * cpw) return;
    const int32_t c = (int32_t)blockIdx.x * cols + (int32_t)threadIdx.x % cols;
    if (c >= nvec) return;
    const int64_t chunk = (int64_t)blockIdx.y * cpw + threadIdx.x / cols;
    const int64_t r0 = chunk * rpc;
    const int64_t r1 = r0 + rpc < M ? r0 + rpc : M;
    float acc[EPV];
#pragma unroll
    for (int k = 0; k < EPV; ++k) acc[k] = 0.f;
    for (int64_t row = r0; row < r1; ++row) {
        const float r = rstd[row];
        float fx[EPV], fg[EPV];
        Elem<T>::unpack(reinterpret_cast<const u32x4 *>(x + row * N)[c], fx);
        Elem<T>::unpack(reinterpret_cast<const u32x4 *>(dy + row * N)[c], fg);
#pragma unroll
        for (int k = 0; k < EPV; ++k) acc[k] = __builtin_fmaf(fg[k] * fx[k], r, acc[k]);
    }
    float4 *dst = reinterpret_cast<float4 *>(partial + chunk * ldp + (int64_t)c * EPV);
#pragma unroll
    for (int q = 0; q < EPV / 4; ++q) dst[q] = make_float4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
}

// ---- the separate residual add -------------------------------------------------

template <typename T>
__global__ void __launch_bounds__(kWG)
un_add(const T *a, const T *b, T *c, int64_t total) {
    constexpr int EPV = Elem<T>::kPerVec;
    const u32x4 *av = reinterpret_cast<const u32x4 *>(a);
    const u32x4 *bv = reinterpret_cast<const u32x4 *>(b);
    u32x4 *cv = reinterpret_cast<u32x4 *>(c);
    for (int64_t i = (int64_t)blockIdx.x * kWG + threadIdx.x; i < total; i += (int64_t)gridDim.x * kWG) {
        float f[EPV], g[EPV];
        Elem<T>::unpack(av[i], f);
        Elem<T>::unpack(bv[i], g);
#pragma unroll
        for (int k = 0; k < EPV; ++k) f[k] += g[k];
        cv[i] = Elem<T>::pack(f);
    }
}

// ---- host ---------------------------------------------------------------------

int esize(int dtype) { return dtype == RMSN_F32 ? 4 : 2; }
bool valid(int dtype) { return dtype >= RMSN_F32 && dtype <= RMSN_F16_WF32; }
bool a16(const void *p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// activation type T and weight type TW of a format, passed as null pointers
template <class F>
int with_types(int dtype, F &&f) {
    switch (dtype) {
    case RMSN_F32: return f((float *)nullptr, (float *)nullptr);
    case RMSN_BF16: return f((bf16_t *)nullptr, (bf16_t *)nullptr);
    case RMSN_F16: return f((f16_t *)nullptr, (f16_t *)nullptr);
    case RMSN_BF16_WF32: return f((bf16_t *)nullptr, (float *)nullptr);
    case RMSN_F16_WF32: return f((f16_t *)nullptr, (float *)nullptr);
    default: return RMSN_EDTYPE;
    }
}

int shape_ok(int64_t M, int64_t N, int dtype) {
    if (!valid(dtype)) return RMSN_EDTYPE;
    if (M < 0 || N < 1 || N > (int64_t(1) << 30) || M > INT64_MAX / N / 4) return RMSN_EINVAL;
    if ((N * esize(dtype)) % 16 != 0) return RMSN_EINVAL;
    return RMSN_OK;
}

unsigned grid_of(int64_t items, int64_t per_wg) {
    int64_t g = (items + per_wg - 1) / per_wg;
    return (unsigned)(g < 1 ? 1 : (g > kMaxGrid ? kMaxGrid : g));
}

int status(hipError_t e) { return e == hipSuccess ? RMSN_OK : RMSN_EHIP; }

// vectors per workgroup of the dW column kernel, and its row-chunk count:
// at least kPartialRows chunks (fewer when M is smaller), more for narrow
// rows so that about 64K lanes work, rounded up to whole workgroups
int64_t dw_cols(int64_t nvec) { return nvec < kWG ? nvec : kWG; }
int64_t chunks(int64_t M, int64_t nvec) {
    const int64_t cpw = kWG / dw_cols(nvec);
    int64_t want = (int64_t(1) << 16) / nvec;
    want = want < kPartialRows ? kPartialRows : want;
    want = want < M ? want : M;
    return (want + cpw - 1) / cpw * cpw;
}
int64_t stride(int64_t N) { return (N + kAlign - 1) / kAlign * kAlign; }
int64_t s_offset(int64_t M, int64_t N, int64_t nvec) { return chunks(M, nvec) * stride(N) * 4; }

}  // namespace rmsn_base

using namespace rmsn_base;

extern "C" {

int rmsn_unfused_fwd(const void *x, const void *w, float eps, int64_t M, int64_t N, int dtype, void *y,
                     float *rstd, void *stream) {
    int st = shape_ok(M, N, dtype);
    if (st != RMSN_OK) return st;
    if (!(eps >= 0.f) || !std::isfinite(eps)) return RMSN_EINVAL;
    if (M == 0) return RMSN_OK;
    if (!a16(x) || !a16(w) || !a16(y) || !rstd) return RMSN_EINVAL;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const int32_t nvec = (int32_t)(N * esize(dtype) / 16), n32 = (int32_t)N;
    const int64_t total = M * (int64_t)nvec;
    return with_types(dtype, [&](auto *t, auto *tw) {
        using T = std::remove_pointer_t<decltype(t)>;
        using TW = std::remove_pointer_t<decltype(tw)>;
        hipLaunchKernelGGL(un_rstd<T>, dim3(grid_of(M, kRowsPerWG)), dim3(kWG), 0, s, static_cast<const T *>(x), eps,
                           M, n32, nvec, rstd);
        hipLaunchKernelGGL((un_scale<T, TW>), dim3(grid_of(total, kWG)), dim3(kWG), 0, s, static_cast<const T *>(x),
                           static_cast<const TW *>(w), (const float *)rstd, static_cast<T *>(y), total, nvec);
        return status(hipGetLastError());
    });
}

int64_t rmsn_unfused_bwd_workspace_bytes(int64_t M, int64_t N, int dtype) {
    int st = shape_ok(M, N, dtype);
    if (st != RMSN_OK) return st;
    if (M == 0) return 0;
    return s_offset(M, N, N * esize(dtype) / 16) + (M * 4 + 255) / 256 * 256;
}

int rmsn_unfused_bwd(const void *x, const void *w, const void *dy, const float *rstd, int64_t M, int64_t N,
                     int dtype, void *dx, float *dw, void *workspace, size_t workspace_bytes, void *stream) {
    int st = shape_ok(M, N, dtype);
    if (st != RMSN_OK) return st;
    if (!dw) return RMSN_EINVAL;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (M == 0) return rmsnorm_bwd_combine(nullptr, 0, N, dw, stream);
    if (!a16(x) || !a16(w) || !a16(dy) || !a16(dx) || !rstd) return RMSN_EINVAL;
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return RMSN_EWORKSPACE;
    if (workspace_bytes < (size_t)rmsn_unfused_bwd_workspace_bytes(M, N, dtype)) return RMSN_EWORKSPACE;
    const int32_t nvec = (int32_t)(N * esize(dtype) / 16), n32 = (int32_t)N;
    const int64_t total = M * (int64_t)nvec;
    const int64_t P = chunks(M, nvec), rpc = (M + P - 1) / P, ldp = stride(N);
    const int32_t cols = (int32_t)dw_cols(nvec);
    float *partial = static_cast<float *>(workspace);
    float *sbuf = reinterpret_cast<float *>(static_cast<char *>(workspace) + s_offset(M, N, nvec));
    st = with_types(dtype, [&](auto *t, auto *tw) {
        using T = std::remove_pointer_t<decltype(t)>;
        using TW = std::remove_pointer_t<decltype(tw)>;
        const T *xp = static_cast<const T *>(x), *gp = static_cast<const T *>(dy);
        const TW *wp = static_cast<const TW *>(w);
        hipLaunchKernelGGL((un_dot<T, TW>), dim3(grid_of(M, kRowsPerWG)), dim3(kWG), 0, s, xp, wp, gp, M, n32, nvec,
                           sbuf);
        hipLaunchKernelGGL((un_dx<T, TW>), dim3(grid_of(total, kWG)), dim3(kWG), 0, s, xp, wp, gp, rstd,
                           (const float *)sbuf, static_cast<T *>(dx), total, nvec, (float)N);
        hipLaunchKernelGGL(un_dw_partial<T>, dim3((unsigned)((nvec + cols - 1) / cols), (unsigned)(P / (kWG / cols))),
                           dim3(kWG), 0, s, xp, gp, rstd, M, n32, nvec, cols, rpc, partial, ldp);
        return status(hipGetLastError());
    });
    if (st != RMSN_OK) return st;
    return rmsnorm_bwd_combine(workspace, P, N, dw, stream);
}

int rmsn_add(const void *a, const void *b, void *c, int64_t n, int dtype, void *stream) {
    if (!valid(dtype)) return RMSN_EDTYPE;
    if (n < 0 || n > INT64_MAX / 4) return RMSN_EINVAL;
    if (n == 0) return RMSN_OK;
    if (!a16(a) || !a16(b) || !a16(c) || (n * esize(dtype)) % 16 != 0) return RMSN_EINVAL;
    const int64_t total = n * esize(dtype) / 16;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    return with_types(dtype, [&](auto *t, auto *) {
        using T = std::remove_pointer_t<decltype(t)>;
        hipLaunchKernelGGL(un_add<T>, dim3(grid_of(total, kWG)), dim3(kWG), 0, s, static_cast<const T *>(a),
                           static_cast<const T *>(b), static_cast<T *>(c), total);
        return status(hipGetLastError());
    });
}

}  // extern "C"
