// rmsn_fwd_loop.h -- forward for rows wider than the vector kernels hold in
// registers (more than 16 16-byte vectors on each of 1024 lanes, or 8 with
// the fused residual add).
//
// The same arithmetic as the vector kernel (hello-gpu "Chapter 13 Fused
// RMSNorm", section 13.1; with RES the residual sum of "Profiling, GPU
// utilisation and writing a fused kernel", Problem 15), in two passes over
// the row, one row per 1024-lane workgroup, CH vectors per lane at a time:
// pass 1 loads each chunk of x (with RES also res, and stores h = round(x +
// res)) and adds its squares; after the row sum, pass 2 scales each chunk by
// rstd and the weights and stores y. A row of 262144 16-bit columns is 512
// KiB, more than a workgroup's registers and LDS hold, so part of the row is
// read twice: the first KV vectors per lane stay in registers from pass 1
// (packed, KV / CH chunks), the next LV in the lane's own LDS slots (LV / CH
// chunks; a lane reads back only what it wrote, so no barrier), both loaded
// with the streaming hint as they are not read again; pass 2 scales the kept
// chunks first, then the held ones, and then loads the rest of the row
// again. Pass 1's loads of that rest carry no streaming hint, so pass 2
// finds it in the caches (a CU's row in the MALL) rather than in HBM. With
// RES, pass 2 recomputes h from x and res (both read-only) instead of
// reading back the h it stored, so no load depends on the ordering of this
// workgroup's own stores.
#pragma once

#include "rmsn_device.h"
#include "rmsn_tables.h"

namespace rmsn {

// the cache-policy bits of a load, as a type (for a generic lambda)
template <int A>
struct LoadAux {
    static constexpr int value = A;
};

template <typename T, typename TW, bool RES, int CH, int WPE, int KV, int LV>
__global__ void __launch_bounds__(kWideLanes) __attribute__((amdgpu_waves_per_eu(WPE)))
fwd_loop(const T *__restrict__ x, const T *__restrict__ res, const TW *__restrict__ w, T *__restrict__ h,
         T *__restrict__ y, float *__restrict__ rstd, float eps, int64_t M, int32_t N, int32_t nvec,
         int32_t /*stream_ld*/) {
    using E = Elem<T>;
    using WV = WeightVec<T, TW>;
    constexpr int LPR = kWideLanes;
    constexpr int EPV = E::kPerVec;
    static_assert(KV % CH == 0 && LV % CH == 0, "whole chunks are kept");
    constexpr int KEEP = KV / CH;           // chunks kept in registers
    constexpr int KC = KEEP > 0 ? KEEP : 1;
    constexpr int HOLD = LV / CH;           // chunks after those held in LDS
    static_assert(LV * LPR * 16 <= kWideLdsBytes, "held chunks fit in LDS");
    __shared__ float slots[2 * (LPR / 64)];
    __shared__ u32x4 held[LV > 0 ? LV * LPR : 1];  // lane l's vector v at v * LPR + l

    const int lane = threadIdx.x;
    const float n = (float)N;
    const uint32_t row_bytes = (uint32_t)nvec * 16u;
    const Buf wb(w, row_bytes * WV::kVecs);
    int parity = 0;
    const int nch = (nvec + CH * LPR - 1) / (CH * LPR);

    // the chunk's vector offsets (kOff past the row end)
    auto chunk_offsets = [&](int c0, uint32_t (&off)[CH]) {
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            const int idx = c0 + k * LPR + lane;
            off[k] = idx < nvec ? (uint32_t)idx * 16u : kOff;
        }
    };
    // the chunk's inputs at vector c0 + v * LPR + lane: v = x, or round(x + res)
    auto load_chunk = [&](const Buf &xb, const Buf &rb, int c0, uint32_t (&off)[CH], u32x4 (&v)[CH], auto aux) {
        constexpr int A = decltype(aux)::value;
        chunk_offsets(c0, off);
#pragma unroll
        for (int k = 0; k < CH; ++k) v[k] = xb.load16<A>(off[k]);
        if constexpr (RES) {
            u32x4 r[CH];
#pragma unroll
            for (int k = 0; k < CH; ++k) r[k] = rb.load16<A>(off[k]);
#pragma unroll
            for (int k = 0; k < CH; ++k) {
                float a[EPV], b[EPV];
                E::unpack(v[k], a);
                E::unpack(r[k], b);
#pragma unroll
                for (int e = 0; e < EPV; ++e) a[e] += b[e];
                v[k] = E::pack(a);
            }
        }
    };

    // y = (v * r) * w for one chunk
    auto finish_chunk = [&](const Buf &yb, float r, int c0, const uint32_t (&off)[CH], const u32x4 (&v)[CH]) {
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            WV t;
            t.load(wb, c0 + k * LPR + lane, off[k] != kOff);
            float f[EPV], g[EPV];
            E::unpack(v[k], f);
            t.unpack(g);
#pragma unroll
            for (int e = 0; e < EPV; ++e) f[e] = (f[e] * r) * g[e];
            yb.store16<RMSN_FWD_STORE_AUX>(off[k], E::pack(f));
        }
    };

    for (int64_t row = blockIdx.x; row < M; row += gridDim.x) {
        const Buf xb(x + row * N, row_bytes);
        const Buf rb(RES ? res + row * N : x, RES ? row_bytes : 0u);
        const Buf hb(RES ? h + row * N : y, RES ? row_bytes : 0u);
        const Buf yb(y + row * N, row_bytes);

        float ss = 0.f;
        u32x4 kept[KC][CH];
        if constexpr (KEEP > 0) {
#pragma unroll
            for (int q = 0; q < KEEP; ++q) {
                uint32_t off[CH];
                load_chunk(xb, rb, q * CH * LPR, off, kept[q], LoadAux<RMSN_FWD_LOAD_AUX>{});
#pragma unroll
                for (int k = 0; k < CH; ++k) {
                    if constexpr (RES) hb.store16<RMSN_FWD_STORE_AUX>(off[k], kept[q][k]);
                    ss = E::sumsq(kept[q][k], ss);
                    keep_packed(kept[q][k]);
                }
            }
        }
        for (int ci = KEEP; ci < nch; ++ci) {
            const int c0 = ci * CH * LPR;
            uint32_t off[CH];
            u32x4 v[CH];
            if (ci < KEEP + HOLD) {
                // held in this lane's own LDS slots for pass 2, so no barrier
                load_chunk(xb, rb, c0, off, v, LoadAux<RMSN_FWD_LOAD_AUX>{});
#pragma unroll
                for (int k = 0; k < CH; ++k) held[((ci - KEEP) * CH + k) * LPR + lane] = v[k];
            } else {
                load_chunk(xb, rb, c0, off, v, LoadAux<RMSN_FWD_NARROW_LOAD_AUX>{});
            }
#pragma unroll
            for (int k = 0; k < CH; ++k) {
                if constexpr (RES) hb.store16<RMSN_FWD_STORE_AUX>(off[k], v[k]);
                ss = E::sumsq(v[k], ss);
            }
        }
        ss = row_sum<LPR, LPR>(ss, slots, parity);
        parity ^= 1;
        const float r = __frsqrt_rn(ss / n + eps);
        if (rstd) {
            const Buf sb(rstd + row, 4u);
            sb.store4(lane == 0 ? 0u : kOff, r);
        }

        if constexpr (KEEP > 0) {
#pragma unroll
            for (int q = 0; q < KEEP; ++q) {
                uint32_t off[CH];
                chunk_offsets(q * CH * LPR, off);
                finish_chunk(yb, r, q * CH * LPR, off, kept[q]);
            }
        }
        for (int ci = KEEP; ci < nch; ++ci) {
            const int c0 = ci * CH * LPR;
            uint32_t off[CH];
            u32x4 v[CH];
            if (ci < KEEP + HOLD) {
                chunk_offsets(c0, off);
#pragma unroll
                for (int k = 0; k < CH; ++k) v[k] = held[((ci - KEEP) * CH + k) * LPR + lane];
            } else {
                load_chunk(xb, rb, c0, off, v, LoadAux<RMSN_FWD_LOAD_AUX>{});
            }
            finish_chunk(yb, r, c0, off, v);
        }
    }
}

}  // namespace rmsn
