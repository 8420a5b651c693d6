// rmsn_common.hip -- the kernels that do not depend on the vector shape: the
// scalar (any-N) forward and backward row kernels, the fixed-order dW combine
// and a zero fill; plus the dtype dispatch of the vector-kernel tables.
#include "rmsn_bwd_kernels.h"
#include "rmsn_fwd_kernels.h"

namespace rmsn {

// dW[col] = sum over p of partial[p][col]. A workgroup of kCombineWG lanes
// takes Q = kCombineWG / S lanes per slice and 4 Q columns (each partial row
// contributes whole 128-byte cache lines to one workgroup only; narrower
// strips made two workgroups, usually on different XCDs, fetch the same
// line). Lane (slice s, quad c) sums rows p = s, s + S, s + 2S, ... in
// ascending order for columns 4c..4c+3; the S slice sums are then folded by a
// fixed binary tree in LDS. A lane issues the loads of kCombineUnroll of its
// rows before adding them (still in ascending order), so the partial rows
// stream in with that many loads in flight per lane instead of one memory
// latency per row. S is chosen by the host from P and N (fewer slices give
// fewer, wider workgroups); for a given S the order is fixed, so dW is
// bit-identical from run to run. Rows are padded to ldp floats (a multiple of
// 64) and 256-byte aligned, so the float4 loads stay inside the workspace.
template <int S>
__global__ void __launch_bounds__(kCombineWG)
dw_combine(const float *__restrict__ partial, int64_t ldp, int64_t P, int32_t N, float *__restrict__ dw) {
    constexpr int Q = kCombineWG / S;
    static_assert(Q * S == kCombineWG && Q >= 8, "whole 128-byte lines per slice");
    __shared__ double4 red[S][Q];
    const int quad = threadIdx.x % Q;
    const int slice = threadIdx.x / Q;
    const int64_t col = (int64_t)blockIdx.x * (4 * Q) + 4 * quad;
    double4 a = make_double4(0.0, 0.0, 0.0, 0.0);
    if (col < N) {
        constexpr int U = kCombineUnroll;
        int64_t p = slice;
        for (; p + (U - 1) * S < P; p += U * S) {
            float4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = *reinterpret_cast<const float4 *>(partial + (p + u * S) * ldp + col);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                a.x += (double)v[u].x;
                a.y += (double)v[u].y;
                a.z += (double)v[u].z;
                a.w += (double)v[u].w;
            }
        }
        for (; p < P; p += S) {
            const float4 v = *reinterpret_cast<const float4 *>(partial + p * ldp + col);
            a.x += (double)v.x;
            a.y += (double)v.y;
            a.z += (double)v.z;
            a.w += (double)v.w;
        }
    }
    red[slice][quad] = a;
    __syncthreads();
#pragma unroll
    for (int h = S / 2; h >= 1; h >>= 1) {
        if (slice < h) {
            double4 u = red[slice][quad];
            const double4 v = red[slice + h][quad];
            u.x += v.x;
            u.y += v.y;
            u.z += v.z;
            u.w += v.w;
            red[slice][quad] = u;
        }
        __syncthreads();
    }
    if (slice == 0 && col < N) {
        const double4 u = red[0][quad];
        const float o[4] = {(float)u.x, (float)u.y, (float)u.z, (float)u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (col + e < N) dw[col + e] = o[e];
    }
}

__global__ void __launch_bounds__(256) fill_zero(float *__restrict__ p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.f;
}

#define RMSN_FORMATS(X) X(f32) X(bf16) X(f16) X(bf16w32) X(f16w32)
#define RMSN_DECL(tag)                                                                 \
    const KernelEntry *fwd_vec_kernel_##tag(int res, int lpr, int vpt, int wg, int pf); \
    const KernelEntry *bwd_vec_kernel_##tag(int res, int lpr, int vpt, int wg, int pf); \
    const KernelEntry *bwd_wide_kernel_##tag(int res, int vpt, int pf);                  \
    const KernelEntry *bwd_lds_kernel_##tag(int res, int lpr, int wg, int st);           \
    const KernelEntry *bwd_wide_lds_kernel_##tag(int lpr, int vpt, int st);            \
    const KernelEntry *bwd_split_kernel_##tag(int res, int vpt, int pf);               \
    const KernelEntry *fwd_loop_kernel_##tag(int res, int ch, int kv, int lv);
RMSN_FORMATS(RMSN_DECL)
#undef RMSN_DECL

// Format codes (rmsn_dtype): 0 fp32, 1 bf16, 2 fp16, 3 bf16 with fp32 weights,
// 4 fp16 with fp32 weights.
const KernelEntry *fwd_vec_kernel(int dtype, int res, int lpr, int vpt, int wg, int pf) {
    switch (dtype) {
    case 0: return fwd_vec_kernel_f32(res, lpr, vpt, wg, pf);
    case 1: return fwd_vec_kernel_bf16(res, lpr, vpt, wg, pf);
    case 2: return fwd_vec_kernel_f16(res, lpr, vpt, wg, pf);
    case 3: return fwd_vec_kernel_bf16w32(res, lpr, vpt, wg, pf);
    case 4: return fwd_vec_kernel_f16w32(res, lpr, vpt, wg, pf);
    default: return nullptr;
    }
}

const KernelEntry *bwd_vec_kernel(int dtype, int res, int lpr, int vpt, int wg, int pf) {
    switch (dtype) {
    case 0: return bwd_vec_kernel_f32(res, lpr, vpt, wg, pf);
    case 1: return bwd_vec_kernel_bf16(res, lpr, vpt, wg, pf);
    case 2: return bwd_vec_kernel_f16(res, lpr, vpt, wg, pf);
    case 3: return bwd_vec_kernel_bf16w32(res, lpr, vpt, wg, pf);
    case 4: return bwd_vec_kernel_f16w32(res, lpr, vpt, wg, pf);
    default: return nullptr;
    }
}

const KernelEntry *bwd_wide_kernel(int dtype, int res, int vpt, int pf) {
    switch (dtype) {
    case 0: return bwd_wide_kernel_f32(res, vpt, pf);
    case 1: return bwd_wide_kernel_bf16(res, vpt, pf);
    case 2: return bwd_wide_kernel_f16(res, vpt, pf);
    case 3: return bwd_wide_kernel_bf16w32(res, vpt, pf);
    case 4: return bwd_wide_kernel_f16w32(res, vpt, pf);
    default: return nullptr;
    }
}

const KernelEntry *bwd_lds_kernel(int dtype, int res, int lpr, int wg, int st) {
    switch (dtype) {
    case 0: return bwd_lds_kernel_f32(res, lpr, wg, st);
    case 1: return bwd_lds_kernel_bf16(res, lpr, wg, st);
    case 2: return bwd_lds_kernel_f16(res, lpr, wg, st);
    case 3: return bwd_lds_kernel_bf16w32(res, lpr, wg, st);
    case 4: return bwd_lds_kernel_f16w32(res, lpr, wg, st);
    default: return nullptr;
    }
}

const KernelEntry *fwd_loop_kernel(int dtype, int res, int ch, int kv, int lv) {
    switch (dtype) {
    case 0: return fwd_loop_kernel_f32(res, ch, kv, lv);
    case 1: return fwd_loop_kernel_bf16(res, ch, kv, lv);
    case 2: return fwd_loop_kernel_f16(res, ch, kv, lv);
    case 3: return fwd_loop_kernel_bf16w32(res, ch, kv, lv);
    case 4: return fwd_loop_kernel_f16w32(res, ch, kv, lv);
    default: return nullptr;
    }
}

const KernelEntry *bwd_split_kernel(int dtype, int res, int vpt, int pf) {
    switch (dtype) {
    case 0: return bwd_split_kernel_f32(res, vpt, pf);
    case 1: return bwd_split_kernel_bf16(res, vpt, pf);
    case 2: return bwd_split_kernel_f16(res, vpt, pf);
    case 3: return bwd_split_kernel_bf16w32(res, vpt, pf);
    case 4: return bwd_split_kernel_f16w32(res, vpt, pf);
    default: return nullptr;
    }
}

const KernelEntry *bwd_wide_lds_kernel(int dtype, int lpr, int vpt, int st) {
    switch (dtype) {
    case 0: return bwd_wide_lds_kernel_f32(lpr, vpt, st);
    case 1: return bwd_wide_lds_kernel_bf16(lpr, vpt, st);
    case 2: return bwd_wide_lds_kernel_f16(lpr, vpt, st);
    case 3: return bwd_wide_lds_kernel_bf16w32(lpr, vpt, st);
    case 4: return bwd_wide_lds_kernel_f16w32(lpr, vpt, st);
    default: return nullptr;
    }
}

template <typename T, typename TW>
const void *scalar_kernel(int is_bwd, int res, int lds) {
    if (is_bwd) {
        if (lds)
            return res ? reinterpret_cast<const void *>(&bwd_scalar<T, TW, true, true>)
                       : reinterpret_cast<const void *>(&bwd_scalar<T, TW, false, true>);
        return res ? reinterpret_cast<const void *>(&bwd_scalar<T, TW, true, false>)
                   : reinterpret_cast<const void *>(&bwd_scalar<T, TW, false, false>);
    }
    return res ? reinterpret_cast<const void *>(&fwd_scalar<T, TW, true>)
               : reinterpret_cast<const void *>(&fwd_scalar<T, TW, false>);
}

const void *scalar_kernel(int dtype, int is_bwd, int res, int lds) {
    switch (dtype) {
    case 0: return scalar_kernel<float, float>(is_bwd, res, lds);
    case 1: return scalar_kernel<bf16_t, bf16_t>(is_bwd, res, lds);
    case 2: return scalar_kernel<f16_t, f16_t>(is_bwd, res, lds);
    case 3: return scalar_kernel<bf16_t, float>(is_bwd, res, lds);
    case 4: return scalar_kernel<f16_t, float>(is_bwd, res, lds);
    default: return nullptr;
    }
}

const void *dw_combine_kernel(int slices) {
    switch (slices) {
    case 8: return reinterpret_cast<const void *>(&dw_combine<8>);
    case 16: return reinterpret_cast<const void *>(&dw_combine<16>);
    case 32: return reinterpret_cast<const void *>(&dw_combine<32>);
    case 64: return reinterpret_cast<const void *>(&dw_combine<64>);
    default: return nullptr;
    }
}
const void *fill_zero_kernel() { return reinterpret_cast<const void *>(&fill_zero); }

}  // namespace rmsn
