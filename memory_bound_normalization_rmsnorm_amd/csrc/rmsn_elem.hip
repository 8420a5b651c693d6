// rmsn_elem.hip -- RMSNorm forward and backward at element granularity, for
// rows the 16-byte vector kernels cannot take: a row whose byte size is not a
// multiple of 16 (e.g. 4100 bf16 columns) or a pointer that is not 16-byte
// aligned. The arithmetic is that of the vector kernels (hello-gpu "Chapter 13
// Fused RMSNorm", section 13.1, for the forward; "RMSNorm backward (almost)
// without the column reduction", section "The backward pass", for dx and dW;
// the fused residual add of the page "Profiling, GPU utilisation and writing
// a fused kernel", Problem 15, read as the unfused composition).
//
// A row is one workgroup of kElemWG lanes; lane l holds elements
// l + k * kElemWG (k < K) in registers, loaded once with element loads (each
// wavefront instruction reads 64 consecutive elements, coalesced whatever the
// row's alignment). Elements past the row end are masked. The forward runs
// one row per workgroup pass over a grid of rows; the backward is persistent
// (a fixed cyclic row -> workgroup map) and keeps its dW running sums in
// registers, writing one fp32 partial row per workgroup for the fixed-order
// combine. No atomics.
#include "rmsn_device.h"
#include "rmsn_tables.h"

namespace rmsn {

template <typename T, typename TW, bool RES, int K>
__global__ void __launch_bounds__(kElemWG)
fwd_elem(const T *__restrict__ x, const T *__restrict__ res, const TW *__restrict__ w, T *__restrict__ h,
         T *__restrict__ y, float *__restrict__ rstd, float eps, int64_t M, int32_t N, int32_t /*nvec*/,
         int32_t /*stream_ld*/) {
    using E = Elem<T>;
    __shared__ float slots[2 * (kElemWG / 64)];
    const float n = (float)N;
    float fw[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int j = (int)threadIdx.x + k * kElemWG;
        fw[k] = j < N ? Elem<TW>::load(w + j) : 0.f;
    }
    int parity = 0;
    for (int64_t row = blockIdx.x; row < M; row += gridDim.x) {
        const int64_t o = row * (int64_t)N;
        float v[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int j = (int)threadIdx.x + k * kElemWG;
            v[k] = j < N ? E::load(x + o + j) : 0.f;
        }
        if constexpr (RES) {
            // h = x + res rounded once to the activation format, stored; the row is h as stored
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const int j = (int)threadIdx.x + k * kElemWG;
                if (j < N) {
                    const float a = v[k] + E::load(res + o + j);
                    E::store(h + o + j, a);
                    v[k] = E::rounded(a);
                }
            }
        }
        float ss = 0.f;
#pragma unroll
        for (int k = 0; k < K; ++k) ss = __builtin_fmaf(v[k], v[k], ss);
        ss = row_sum<kElemWG, kElemWG>(ss, slots, parity);
        parity ^= 1;
        const float r = __frsqrt_rn(ss / n + eps);
        if (threadIdx.x == 0 && rstd) rstd[row] = r;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int j = (int)threadIdx.x + k * kElemWG;
            if (j < N) E::store(y + o + j, (v[k] * r) * fw[k]);
        }
    }
}

template <typename T, typename TW, bool RES, int K>
__global__ void __launch_bounds__(kElemWG)
bwd_elem(const T *__restrict__ x, const TW *__restrict__ w, const T *__restrict__ dy, const T *__restrict__ dh,
         const float *__restrict__ rstd, T *__restrict__ dx, float *__restrict__ partial, int64_t ldp, int64_t M,
         int32_t N, int32_t /*nvec*/) {
    using E = Elem<T>;
    __shared__ float slots[2 * (kElemWG / 64)];
    const float n = (float)N;
    float fw[K], acc[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int j = (int)threadIdx.x + k * kElemWG;
        fw[k] = j < N ? Elem<TW>::load(w + j) : 0.f;
        acc[k] = 0.f;
    }
    int parity = 0;
    for (int64_t row = blockIdx.x; row < M; row += gridDim.x) {
        const int64_t o = row * (int64_t)N;
        const float r = rstd[row];
        float fx[K], fg[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int j = (int)threadIdx.x + k * kElemWG;
            fx[k] = j < N ? E::load(x + o + j) : 0.f;
            fg[k] = j < N ? E::load(dy + o + j) : 0.f;
        }
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < K; ++k) s = __builtin_fmaf(fg[k] * fw[k], fx[k], s);
        s = row_sum<kElemWG, kElemWG>(s, slots, parity);
        parity ^= 1;
        const float c = r * (r * (r * (s / n)));  // r^3 S/N without forming r^3
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int j = (int)threadIdx.x + k * kElemWG;
            if (j < N) {
                float g = __builtin_fmaf(-fx[k], c, r * (fg[k] * fw[k]));
                if constexpr (RES) g += E::load(dh + o + j);
                E::store(dx + o + j, g);
                acc[k] = __builtin_fmaf(fg[k] * fx[k], r, acc[k]);
            }
        }
    }
    float *prow = partial + (int64_t)blockIdx.x * ldp;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int j = (int)threadIdx.x + k * kElemWG;
        if (j < N) prow[j] = acc[k];
    }
}

namespace {

template <typename T, typename TW, int K>
const void *pick(int is_bwd, int res) {
    if (is_bwd)
        return res ? reinterpret_cast<const void *>(&bwd_elem<T, TW, true, K>)
                   : reinterpret_cast<const void *>(&bwd_elem<T, TW, false, K>);
    return res ? reinterpret_cast<const void *>(&fwd_elem<T, TW, true, K>)
               : reinterpret_cast<const void *>(&fwd_elem<T, TW, false, K>);
}

template <typename T, typename TW>
const void *pick_k(int is_bwd, int res, int k) {
    switch (k) {
    case 1: return pick<T, TW, 1>(is_bwd, res);
    case 2: return pick<T, TW, 2>(is_bwd, res);
    case 4: return pick<T, TW, 4>(is_bwd, res);
    case 8: return pick<T, TW, 8>(is_bwd, res);
    case 16: return pick<T, TW, 16>(is_bwd, res);
    default: return nullptr;
    }
}

}  // namespace

// Format codes (rmsn_dtype): 0 fp32, 1 bf16, 2 fp16, 3 bf16 with fp32 weights,
// 4 fp16 with fp32 weights.
const void *elem_kernel(int dtype, int is_bwd, int res, int k) {
    switch (dtype) {
    case 0: return pick_k<float, float>(is_bwd, res, k);
    case 1: return pick_k<bf16_t, bf16_t>(is_bwd, res, k);
    case 2: return pick_k<f16_t, f16_t>(is_bwd, res, k);
    case 3: return pick_k<bf16_t, float>(is_bwd, res, k);
    case 4: return pick_k<f16_t, float>(is_bwd, res, k);
    default: return nullptr;
    }
}

}  // namespace rmsn
