// rmsn_fwd_kernels.h -- RMSNorm forward kernel templates for gfx950.
//
// Per row i: rstd_i = 1/sqrt(sum_j v_ij^2 / N + eps), y_ij = v_ij * rstd_i * w_j
// (hello-gpu "Chapter 13 Fused RMSNorm", section 13.1), where v = x, or with
// the fused residual add (RES; page "Profiling, GPU utilisation and writing a
// fused kernel", Problem 15: the residual sum and its normalisation from
// one kernel) v = h = x + res rounded to the activation format, stored,
// and normalised as stored, so the result is that of the unfused add followed
// by the normalisation. The square, the row sum, the scalar and the scaled
// store happen in one kernel with the row held in registers, so every input
// is read from HBM exactly once (the chapter's section 13.2 notes that fusing
// alone does not guarantee a single read).
//
// Formats: activations T (fp32, bf16, fp16); weights TW = T, or fp32 master
// weights with 16-bit activations.
//
// Vector kernel: a row is shared by LPR lanes; lane l holds the 16-byte
// vectors l, l + LPR, l + 2*LPR, ... (VPT of them), so each load instruction
// of a row group covers LPR * 16 contiguous bytes. Accesses go through a
// buffer resource per row block whose record count covers only the rows that
// exist; vectors past the row end use an out-of-range offset. Such lanes load
// zeros (adding nothing to the sum) and store nothing; the mean always
// divides by the true N. A workgroup of WG lanes (a multiple of LPR, at least
// 256) works on WG / LPR rows at a time and strides over rows by
// grid * (WG / LPR); w is loaded into registers once per workgroup. With PF
// the loads of the next row block are issued before the current block's
// arithmetic (a register double buffer: a persistent grid gives up the
// scheduler's latency hiding across workgroups, so the pipelining is explicit).
//
// Scalar kernel: any N and any alignment; one workgroup of 256 lanes per row,
// element loads, the row re-read (from cache) for the output.
#pragma once

#include "rmsn_device.h"
#include "rmsn_tables.h"

namespace rmsn {

// Whether a lane keeps its weights in registers for the whole kernel: yes up
// to 8 weight vectors; beyond (fp32 weights with 16-bit rows at 5 or more
// vectors per lane) they would not fit beside the row, and are re-read from
// cache (w is a few hundred KiB at most, resident in every XCD's L2) where
// they are used.
template <typename T, typename TW, int VPT>
constexpr bool fwd_keeps_w() {
    return VPT * WeightVec<T, TW>::kVecs <= 8;
}

// 16-byte vectors a lane keeps per row slot: x (and res), the weights, and the
// prefetched copies.
template <typename T, typename TW, bool RES, bool PF, int VPT>
constexpr int fwd_packed_per_slot() {
    constexpr int in = RES ? 2 : 1;
    return in + (fwd_keeps_w<T, TW, VPT>() ? WeightVec<T, TW>::kVecs : 0) + (PF ? in : 0);
}

template <typename T, typename TW, bool RES, int LPR, int VPT, int WG, bool PF>
__global__ void __launch_bounds__(WG)
__attribute__((amdgpu_waves_per_eu(waves_for(VPT * fwd_packed_per_slot<T, TW, RES, PF, VPT>(), 0, VPT, WG,
                                             ((RES || WeightVec<T, TW>::kVecs > 1) ? Elem<T>::kPerVec : 0) +
                                                 (fwd_keeps_w<T, TW, VPT>() ? 0 : 4 * VPT * WeightVec<T, TW>::kVecs)))))
fwd_vec(const T *__restrict__ x, const T *__restrict__ res, const TW *__restrict__ w, T *__restrict__ h,
        T *__restrict__ y, float *__restrict__ rstd, float eps, int64_t M, int32_t N, int32_t nvec,
        int32_t stream_ld) {
    using E = Elem<T>;
    using WV = WeightVec<T, TW>;
    constexpr int RPW = WG / LPR;
    // Row loads carry the non-temporal hint when the host asks for it (long
    // grids of wavefront-wide rows); narrow rows never do.
    const bool nt_loads = LPR >= 64 && stream_ld != 0;
    static_assert(WG % LPR == 0, "workgroup must hold whole row groups");
    __shared__ float slots[LPR > 64 ? 2 * (WG / 64) : 1];
    // Narrow rows (several per wavefront): the workgroup's rstd values are
    // gathered in LDS and written by its first RPW lanes in one coalesced
    // store, instead of one partial store per wavefront (a second store
    // instruction per wavefront that cost 3% at 128 columns).
    constexpr bool kGatherRstd = LPR < 64;
    __shared__ float rsh[kGatherRstd ? 2 * RPW : 1];
    int rpar = 0;

    const int lane = threadIdx.x % LPR;
    const int grp = threadIdx.x / LPR;
    const float n = (float)N;
    const uint32_t row_bytes = (uint32_t)nvec * 16u;

    // Byte offset of each of this lane's vectors inside a row block; vectors
    // past the row end get an out-of-range offset.
    constexpr bool kKeepW = fwd_keeps_w<T, TW, VPT>();
    uint32_t off[VPT];
    const Buf wb(w, row_bytes * WV::kVecs);
    WV wv[kKeepW ? VPT : 1];
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int idx = v * LPR + lane;
        const bool in = idx < nvec;
        off[v] = in ? (uint32_t)grp * row_bytes + (uint32_t)idx * 16u : kOff;
        if constexpr (kKeepW) wv[v].load(wb, idx, in);
    }
    // rows of the block starting at b that exist (0 past the end)
    auto rows_at = [&](int64_t b) -> uint32_t {
        const int64_t left = M - b;
        return left <= 0 ? 0u : (left < RPW ? (uint32_t)left : (uint32_t)RPW);
    };
    // the block's input vectors: x, and the residual when fused
    auto load_block = [&](int64_t b, u32x4 (&xo)[VPT], u32x4 (&ro)[VPT]) {
        const int64_t bb = b < M ? b : 0;
        const uint32_t bytes = rows_at(b) * row_bytes;
        const Buf xb(x + bb * N, bytes);
        const Buf rb(RES ? res + bb * N : x, RES ? bytes : 0u);
        if (nt_loads) {
#pragma unroll
            for (int v = 0; v < VPT; ++v) xo[v] = xb.load16<RMSN_FWD_LOAD_AUX>(off[v]);
            if constexpr (RES) {
#pragma unroll
                for (int v = 0; v < VPT; ++v) ro[v] = rb.load16<RMSN_FWD_LOAD_AUX>(off[v]);
            }
        } else {
#pragma unroll
            for (int v = 0; v < VPT; ++v) xo[v] = xb.load16<RMSN_FWD_NARROW_LOAD_AUX>(off[v]);
            if constexpr (RES) {
#pragma unroll
                for (int v = 0; v < VPT; ++v) ro[v] = rb.load16<RMSN_FWD_NARROW_LOAD_AUX>(off[v]);
            }
        }
    };

    int parity = 0;
    const int64_t step = (int64_t)gridDim.x * RPW;
    int64_t base = (int64_t)blockIdx.x * RPW;
    u32x4 xn[VPT], rn[VPT];  // prefetched next block (PF)
    if constexpr (PF) load_block(base, xn, rn);
    for (; base < M; base += step) {
        const uint32_t rows = rows_at(base);
        const Buf yb(y + base * N, rows * row_bytes);

        // The row loads go out before the weights are pinned (pinning waits
        // for the weight loads; issued first, the row loads overlap them) up
        // to 128 lanes per row (5% at 128 columns, 1.6% at 4096), and at any
        // width in the plain forward with 16-bit weights (2-6% at 12288-16384
        // columns, neutral elsewhere). fp32 weights on wider rows pin first:
        // rows first measured 4% slower there (32768 x 8192, 16384 x 16384).
        constexpr bool kRowsFirst = LPR <= 128 || (sizeof(TW) == 2 && !RES);
        if constexpr (kKeepW && !kRowsFirst) {
#pragma unroll
            for (int v = 0; v < VPT; ++v) wv[v].keep();
        }
        u32x4 xv[VPT], rv[VPT];
        if constexpr (PF) {
#pragma unroll
            for (int v = 0; v < VPT; ++v) {
                xv[v] = xn[v];
                if constexpr (RES) rv[v] = rn[v];
            }
            load_block(base + step, xn, rn);
        } else {
            load_block(base, xv, rv);
        }
        if constexpr (kKeepW && kRowsFirst) {
#pragma unroll
            for (int v = 0; v < VPT; ++v) wv[v].keep();
        }
        if constexpr (RES) {
            // h = round(x + res) in the activation format, stored; from here on
            // the row is h as stored
            const Buf hb(h + base * N, rows * row_bytes);
#pragma unroll
            for (int v = 0; v < VPT; ++v) {
                float a[E::kPerVec], b[E::kPerVec];
                E::unpack(xv[v], a);
                E::unpack(rv[v], b);
#pragma unroll
                for (int k = 0; k < E::kPerVec; ++k) a[k] += b[k];
                xv[v] = E::pack(a);
                hb.store16<RMSN_FWD_STORE_AUX>(off[v], xv[v]);
            }
        }

        float ss = 0.f;
#pragma unroll
        for (int v = 0; v < VPT; ++v) ss = E::sumsq(xv[v], ss);
        ss = row_sum<LPR, WG>(ss, slots, parity);
        parity ^= 1;
        const float r = __frsqrt_rn(ss / n + eps);

        if (rstd) {
            const Buf rb(rstd + base, rows * 4u);
            if constexpr (kGatherRstd) {
                // double-buffered: a buffer is rewritten two blocks later, after
                // every lane has passed the next block's barrier
                float *buf = rsh + rpar * RPW;
                if (lane == 0) buf[grp] = r;
                __syncthreads();
                if (threadIdx.x < RPW) rb.store4((uint32_t)threadIdx.x * 4u, buf[threadIdx.x]);
                rpar ^= 1;
            } else {
                rb.store4(lane == 0 ? (uint32_t)grp * 4u : kOff, r);
            }
        }
#pragma unroll
        for (int v = 0; v < VPT; ++v) keep_packed(xv[v]);
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            float f[E::kPerVec], g[E::kPerVec];
            E::unpack(xv[v], f);
            if constexpr (kKeepW) {
                wv[v].unpack(g);
            } else {
                WV t;
                t.load(wb, v * LPR + lane, off[v] != kOff);
                t.unpack(g);
            }
#pragma unroll
            for (int k = 0; k < E::kPerVec; ++k) f[k] = (f[k] * r) * g[k];
            yb.store16<RMSN_FWD_STORE_AUX>(off[v], E::pack(f));
        }
    }
}

template <typename T, typename TW, bool RES>
__global__ void __launch_bounds__(kScalarWG)
fwd_scalar(const T *__restrict__ x, const T *__restrict__ res, const TW *__restrict__ w, T *__restrict__ h,
           T *__restrict__ y, float *__restrict__ rstd, float eps, int64_t M, int32_t N, int32_t /*nvec*/,
           int32_t /*stream_ld*/) {
    using E = Elem<T>;
    __shared__ float slots[2 * (kScalarWG / 64)];
    const float n = (float)N;
    int parity = 0;
    for (int64_t row = blockIdx.x; row < M; row += gridDim.x) {
        const int64_t o = row * (int64_t)N;
        // the normalised input: x, or the stored sum (written here, re-read below)
        const T *vr = RES ? h + o : x + o;
        float ss = 0.f;
        for (int j = threadIdx.x; j < N; j += kScalarWG) {
            float f = E::load(x + o + j);
            if constexpr (RES) {
                E::store(h + o + j, f + E::load(res + o + j));
                f = E::load(h + o + j);
            }
            ss = __builtin_fmaf(f, f, ss);
        }
        ss = row_sum<kScalarWG, kScalarWG>(ss, slots, parity);
        parity ^= 1;
        const float r = __frsqrt_rn(ss / n + eps);
        if (threadIdx.x == 0 && rstd) rstd[row] = r;
        for (int j = threadIdx.x; j < N; j += kScalarWG)
            E::store(y + o + j, (E::load(vr + j) * r) * Elem<TW>::load(w + j));
    }
}

}  // namespace rmsn
