// rmsn_elem_kernels.h -- RMSNorm forward and backward for rows the 16-byte vector
// kernels cannot take: a row whose byte size is not a multiple of 16 (e.g.
// 4100 bf16 columns) or a pointer that is not 16-byte aligned. The arithmetic
// is that of the vector kernels (hello-gpu "Chapter 13 Fused RMSNorm",
// section 13.1, for the forward; "RMSNorm backward (almost) without the column
// reduction", section "The backward pass", for dx and dW; the fused residual
// add of the page "Profiling, GPU utilisation and writing a fused kernel",
// Problem 15, read as the unfused composition).
//
// Each access moves a group of G consecutive elements (2 to 16 bytes), G the
// largest power of two that divides N and whose bytes divide the alignment of
// every pointer, so that every access is naturally aligned and no row has a
// partial group (4100 bf16 columns: G = 4, 8-byte accesses; 4095: G = 1). A
// row is one workgroup of L lanes (64 to 1024); lane l holds groups l + k * L
// (k < K) in registers, read once; each wavefront access covers 64
// consecutive groups. Groups past the row end are masked. Workgroups walk
// rows cyclically (row = workgroup + t * grid); the backward keeps its dW
// running sums in registers over its rows and writes one fp32 partial row per
// workgroup for the fixed-order combine. No atomics. K * G (elements per
// lane) is the smallest multiple of G that covers the row: registers, and
// with them the workgroups a compute unit holds, grow with it.
#pragma once

#include <type_traits>

#include "rmsn_device.h"
#include "rmsn_tables.h"

namespace rmsn {

// G consecutive elements held as 32-bit words, as they are stored: 4-byte
// elements one per word, 16-bit elements two per word (a lone one in the low
// half). Rows stay packed in registers and are widened where used, so 16-bit
// rows take half the registers of fp32 ones, which keeps two workgroups per
// compute unit at more elements per lane.
template <typename T, int G>
struct Packed {
    static constexpr int kBytes = G * (int)sizeof(T);
    static constexpr int kWords = (kBytes + 3) / 4;
    struct alignas(kBytes) Access {
        uint32_t w[kWords];
    };
    uint32_t w[kWords];

    // one naturally aligned access of G elements
    __device__ __forceinline__ void load(const T *p) {
        if constexpr (kBytes >= 4) {
            const Access a = *reinterpret_cast<const Access *>(p);
#pragma unroll
            for (int i = 0; i < kWords; ++i) w[i] = a.w[i];
        } else {
            w[0] = *reinterpret_cast<const uint16_t *>(p);
        }
    }
    __device__ __forceinline__ void store(T *p) const {
        if constexpr (kBytes >= 4) {
            Access a;
#pragma unroll
            for (int i = 0; i < kWords; ++i) a.w[i] = w[i];
            *reinterpret_cast<Access *>(p) = a;
        } else {
            *reinterpret_cast<uint16_t *>(p) = (uint16_t)w[0];
        }
    }
    __device__ __forceinline__ void clear() {
#pragma unroll
        for (int i = 0; i < kWords; ++i) w[i] = 0u;
    }
    // Hides the words' values from the compiler at this point, so that what
    // was widened from them before is widened again after rather than kept in
    // extra registers (a few ALU operations per element; the kernels wait on
    // memory).
    __device__ __forceinline__ void rewiden() {
#pragma unroll
        for (int i = 0; i < kWords; ++i) asm volatile("" : "+v"(w[i]));
    }
    // element i widened to fp32 (i a compile-time index after unrolling)
    __device__ __forceinline__ float get(int i) const {
        if constexpr (sizeof(T) == 4) {
            return as_float(w[i]);
        } else if constexpr (std::is_same<T, bf16_t>::value) {
            return (i & 1) ? bf16_hi(w[i / 2]) : bf16_lo(w[i / 2]);
        } else {
            return (i & 1) ? f16_hi(w[i / 2]) : f16_lo(w[i / 2]);
        }
    }
    // G fp32 values rounded once to the storage format (round to nearest even)
    __device__ __forceinline__ void set(const float *f) {
        if constexpr (sizeof(T) == 4) {
#pragma unroll
            for (int i = 0; i < G; ++i) w[i] = as_u32(f[i]);
        } else if constexpr (G == 1) {
            T e;
            Elem<T>::store(&e, f[0]);
            w[0] = e.bits;
        } else {
#pragma unroll
            for (int i = 0; i < kWords; ++i)
                w[i] = std::is_same<T, bf16_t>::value ? pack_bf16x2(f[2 * i], f[2 * i + 1])
                                                      : pack_f16x2(f[2 * i], f[2 * i + 1]);
        }
    }
};

// The lane's groups of one row (zeros past the row end).
template <typename T, int L, int K, int G>
__device__ __forceinline__ void load_row(const T *__restrict__ p, int32_t N, Packed<T, G> (&v)[K]) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int j = G * ((int)threadIdx.x + k * L);
        if (j < N)
            v[k].load(p + j);
        else
            v[k].clear();
    }
}

template <typename T, typename TW, bool RES, int L, int K, int G>
__global__ void __launch_bounds__(L)
fwd_elem(const T *__restrict__ x, const T *__restrict__ res, const TW *__restrict__ w, T *__restrict__ h,
         T *__restrict__ y, float *__restrict__ rstd, float eps, int64_t M, int32_t N, int32_t /*nvec*/,
         int32_t /*stream_ld*/) {
    __shared__ float slots[2 * (L / 64)];
    const float n = (float)N;
    Packed<TW, G> gw[K];
    load_row<TW, L, K, G>(w, N, gw);
    int parity = 0;
    for (int64_t row = blockIdx.x; row < M; row += gridDim.x) {
        const int64_t o = row * (int64_t)N;
        Packed<T, G> v[K];
        load_row<T, L, K, G>(x + o, N, v);
        if constexpr (RES) {
            // h = x + res rounded once to the activation format and stored; the row is h as stored
            Packed<T, G> q[K];
            load_row<T, L, K, G>(res + o, N, q);
#pragma unroll
            for (int k = 0; k < K; ++k) {
                float a[G];
#pragma unroll
                for (int i = 0; i < G; ++i) a[i] = v[k].get(i) + q[k].get(i);
                v[k].set(a);
                const int j = G * ((int)threadIdx.x + k * L);
                if (j < N) v[k].store(h + o + j);
            }
        }
        float ss = 0.f;
#pragma unroll
        for (int k = 0; k < K; ++k)
#pragma unroll
            for (int i = 0; i < G; ++i) ss = __builtin_fmaf(v[k].get(i), v[k].get(i), ss);
        ss = row_sum<L, L>(ss, slots, parity);
        parity ^= 1;
        const float r = __frsqrt_rn(ss / n + eps);
        if (threadIdx.x == 0 && rstd) rstd[row] = r;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            v[k].rewiden();
            gw[k].rewiden();
            const int j = G * ((int)threadIdx.x + k * L);
            if (j < N) {
                float out[G];
#pragma unroll
                for (int i = 0; i < G; ++i) out[i] = (v[k].get(i) * r) * gw[k].get(i);
                Packed<T, G> o16;
                o16.set(out);
                o16.store(y + o + j);
            }
        }
    }
}

template <typename T, typename TW, bool RES, int L, int K, int G>
__global__ void __launch_bounds__(L)
bwd_elem(const T *__restrict__ x, const TW *__restrict__ w, const T *__restrict__ dy, const T *__restrict__ dh,
         const float *__restrict__ rstd, T *__restrict__ dx, float *__restrict__ partial, int64_t ldp, int64_t M,
         int32_t N, int32_t /*nvec*/) {
    __shared__ float slots[2 * (L / 64)];
    const float n = (float)N;
    Packed<TW, G> gw[K];
    DwSums<K * G, true> acc;  // sum k * G + i: element i of the lane's access k (at most 12)
    load_row<TW, L, K, G>(w, N, gw);
    acc.init();
    int parity = 0;
    Packed<T, G> gx[K], gg[K];  // the row's x and dy
    float r = 0.f;              // and rstd
    if (blockIdx.x < M) {
        load_row<T, L, K, G>(x + blockIdx.x * (int64_t)N, N, gx);
        load_row<T, L, K, G>(dy + blockIdx.x * (int64_t)N, N, gg);
        r = rstd[blockIdx.x];
    }
    for (int64_t row = blockIdx.x; row < M; row += gridDim.x) {
        const int64_t o = row * (int64_t)N;
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            gw[k].rewiden();
#pragma unroll
            for (int i = 0; i < G; ++i) s = __builtin_fmaf(gg[k].get(i) * gw[k].get(i), gx[k].get(i), s);
        }
        s = row_sum<L, L>(s, slots, parity);
        parity ^= 1;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            gx[k].rewiden();
            gg[k].rewiden();
            gw[k].rewiden();
        }
        const float c = r * (r * (r * (s / n)));  // r^3 S/N without forming r^3
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int j = G * ((int)threadIdx.x + k * L);
            if (j < N) {
                float g[G];
                Packed<T, G> d;
                if constexpr (RES) d.load(dh + o + j);  // read here rather than held with x and dy
#pragma unroll
                for (int i = 0; i < G; ++i) {
                    const float fx = gx[k].get(i), fg = gg[k].get(i);
                    g[i] = __builtin_fmaf(-fx, c, r * (fg * gw[k].get(i)));
                    if constexpr (RES) g[i] += d.get(i);
                    acc.add(k * G + i, fg * fx, r);
                }
                Packed<T, G> out;
                out.set(g);
                out.store(dx + o + j);
            }
        }
        acc.end_row();
        const int64_t next = row + gridDim.x;
        if (next < M) {
            load_row<T, L, K, G>(x + next * (int64_t)N, N, gx);
            load_row<T, L, K, G>(dy + next * (int64_t)N, N, gg);
            r = rstd[next];
        }
    }
    // the partial row is 256-byte aligned (or dW itself, 16-byte aligned):
    // stores of up to 4 floats
    constexpr int PG = G < 4 ? G : 4;
    acc.fold();
    float *prow = partial + (int64_t)blockIdx.x * ldp;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int j = G * ((int)threadIdx.x + k * L);
        if (j < N) {
#pragma unroll
            for (int i = 0; i < G; i += PG) {
                float t[PG];
#pragma unroll
                for (int e = 0; e < PG; ++e) t[e] = acc.get(k * G + i + e);
                Packed<float, PG> a;
                a.set(t);
                a.store(prow + j + i);
            }
        }
    }
}

// The kernel of (format, direction, residual, k accesses, g elements per
// access) at L lanes per row; nullptr where none is built. Explicitly
// instantiated once per L, each in its own translation unit.
template <typename T, typename TW, int L, int K, int G>
const void *elem_pick_fn(int is_bwd, int res) {
    if constexpr (K * G > kElemMaxK || G * sizeof(T) > 16 || G * sizeof(TW) > 16) {
        return nullptr;
    } else {
        if (is_bwd)
            return res ? reinterpret_cast<const void *>(&bwd_elem<T, TW, true, L, K, G>)
                       : reinterpret_cast<const void *>(&bwd_elem<T, TW, false, L, K, G>);
        return res ? reinterpret_cast<const void *>(&fwd_elem<T, TW, true, L, K, G>)
                   : reinterpret_cast<const void *>(&fwd_elem<T, TW, false, L, K, G>);
    }
}

template <typename T, typename TW, int L, int G>
const void *elem_pick_k(int is_bwd, int res, int k) {
    switch (k) {
    case 1: return elem_pick_fn<T, TW, L, 1, G>(is_bwd, res);
    case 2: return elem_pick_fn<T, TW, L, 2, G>(is_bwd, res);
    case 3: return elem_pick_fn<T, TW, L, 3, G>(is_bwd, res);
    case 4: return elem_pick_fn<T, TW, L, 4, G>(is_bwd, res);
    case 5: return elem_pick_fn<T, TW, L, 5, G>(is_bwd, res);
    case 6: return elem_pick_fn<T, TW, L, 6, G>(is_bwd, res);
    case 7: return elem_pick_fn<T, TW, L, 7, G>(is_bwd, res);
    case 8: return elem_pick_fn<T, TW, L, 8, G>(is_bwd, res);
    case 9: return elem_pick_fn<T, TW, L, 9, G>(is_bwd, res);
    case 10: return elem_pick_fn<T, TW, L, 10, G>(is_bwd, res);
    case 11: return elem_pick_fn<T, TW, L, 11, G>(is_bwd, res);
    case 12: return elem_pick_fn<T, TW, L, 12, G>(is_bwd, res);
    case 13: return elem_pick_fn<T, TW, L, 13, G>(is_bwd, res);
    case 14: return elem_pick_fn<T, TW, L, 14, G>(is_bwd, res);
    case 15: return elem_pick_fn<T, TW, L, 15, G>(is_bwd, res);
    case 16: return elem_pick_fn<T, TW, L, 16, G>(is_bwd, res);
    default: return nullptr;
    }
}

template <typename T, typename TW, int L>
const void *elem_pick_g(int is_bwd, int res, int k, int g) {
    switch (g) {
    case 1: return elem_pick_k<T, TW, L, 1>(is_bwd, res, k);
    case 2: return elem_pick_k<T, TW, L, 2>(is_bwd, res, k);
    case 4: return elem_pick_k<T, TW, L, 4>(is_bwd, res, k);
    case 8: return elem_pick_k<T, TW, L, 8>(is_bwd, res, k);
    default: return nullptr;
    }
}

// Format codes (rmsn_dtype): 0 fp32, 1 bf16, 2 fp16, 3 bf16 with fp32 weights,
// 4 fp16 with fp32 weights.
template <int L>
const void *elem_pick(int dtype, int is_bwd, int res, int k, int g) {
    switch (dtype) {
    case 0: return elem_pick_g<float, float, L>(is_bwd, res, k, g);
    case 1: return elem_pick_g<bf16_t, bf16_t, L>(is_bwd, res, k, g);
    case 2: return elem_pick_g<f16_t, f16_t, L>(is_bwd, res, k, g);
    case 3: return elem_pick_g<bf16_t, float, L>(is_bwd, res, k, g);
    case 4: return elem_pick_g<f16_t, float, L>(is_bwd, res, k, g);
    default: return nullptr;
    }
}

extern template const void *elem_pick<64>(int, int, int, int, int);
extern template const void *elem_pick<128>(int, int, int, int, int);
extern template const void *elem_pick<256>(int, int, int, int, int);
extern template const void *elem_pick<512>(int, int, int, int, int);
extern template const void *elem_pick<1024>(int, int, int, int, int);

}  // namespace rmsn
