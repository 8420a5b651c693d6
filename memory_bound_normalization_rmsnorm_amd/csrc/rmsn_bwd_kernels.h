// rmsn_bwd_kernels.h -- RMSNorm backward kernel templates for gfx950.
//
// Per row i, with r = rstd_i (written by the forward), V_ij = dy_ij * w_j
// and S_i = sum_j V_ij x_ij:
//     dx_ij = r V_ij - x_ij r^3 S_i / N,    dW_j = sum_i dy_ij x_ij r_i
// ("RMSNorm backward (almost) without the column reduction": the formulas of
// section "The backward pass", the persistent design of section "The
// persistent kernel"). With the fused residual add (RES), x is the stored sum
// h the forward wrote and the gradient dh flowing into h from the residual
// branch is added before the single rounding: dx = dh + (the dx above), the
// gradient of both inputs of the sum.
//
// Persistent row kernel: the grid is sized to what the chip keeps resident.
// Workgroup b works on rows b*RPW .. b*RPW+RPW-1, then strides by grid*RPW, a
// fixed row -> workgroup map. Each lane keeps running dW sums for its columns
// in registers over all the rows it visits; at the end the RPW row groups of
// the workgroup are added in group order through LDS and the workgroup writes
// one fp32 partial row. No atomics anywhere. With PF the next row block's
// loads are issued before the current block's arithmetic (a register double
// buffer in place of the pages' shared-memory async-copy pipeline: the
// persistent grid gives up the scheduler's latency hiding).
//
// The results depend only on (M, N, dtype, grid): the same call on the same
// device gives the same bits every time.
#pragma once

#include "rmsn_device.h"
#include "rmsn_tables.h"

namespace rmsn {

// 16-byte vectors a lane keeps per row slot: x, dy (and dh), the weights, and
// the PF prefetched copies.
template <typename T, typename TW, bool RES, int PF>
constexpr int bwd_packed_per_slot() {
    constexpr int in = RES ? 3 : 2;
    return in * (1 + PF) + WeightVec<T, TW>::kVecs;
}

// Registers beyond the packed vectors that bwd_vec's estimate counts: the
// residual's and the second prefetch slot's unpacked temporaries.
template <typename T, bool RES, int PF>
constexpr int bwd_vec_extra() {
    return (RES ? 2 * Elem<T>::kPerVec : 0) + (PF == 2 ? 2 * Elem<T>::kPerVec : 0);
}

// Whether bwd_vec keeps fp64 dW totals (DwSums): at most 8 sums per lane, and
// only where they cost no resident workgroup: with two blocks prefetched (the
// ladder runs those one per CU), or where the occupancy target still admits
// two workgroups per CU. Elsewhere (1024-lane workgroups without deep
// prefetch, which the ladder may run two per CU) the sums stay fp32.
template <typename T, typename TW, bool RES, int VPT, int WG, int PF>
constexpr bool bwd_vec_dw_f64() {
    constexpr int nv = VPT * Elem<T>::kPerVec;
    if (nv > 8) return false;
    if (PF == 2) return true;
    constexpr int two = 2 * WG / 256 < 8 ? 2 * WG / 256 : 8;
    return waves_for(VPT * bwd_packed_per_slot<T, TW, RES, PF>(), dw_sum_regs(nv, true), VPT, WG,
                     bwd_vec_extra<T, RES, PF>()) >= two;
}

// PF: row blocks loaded ahead of the one being computed (0, 1 or 2; a
// register ring, the loop unrolled so every slot index is static).
// LPR = 0: the row is the whole workgroup, whose size (a multiple of 64 up to
// WG) is chosen at launch, so a row of 640 or 896 vectors runs on 10 or 14
// wavefronts with every lane holding a vector (one vector per lane).
template <typename T, typename TW, bool RES, int LPR, int VPT, int WG, int PF>
__global__ void __launch_bounds__(WG)
__attribute__((amdgpu_waves_per_eu(waves_for(VPT * bwd_packed_per_slot<T, TW, RES, PF>(),
                                             dw_sum_regs(VPT * Elem<T>::kPerVec,
                                                         bwd_vec_dw_f64<T, TW, RES, VPT, WG, PF>()),
                                             VPT, WG, bwd_vec_extra<T, RES, PF>()))))
bwd_vec(const T *__restrict__ x, const TW *__restrict__ w, const T *__restrict__ dy, const T *__restrict__ dh,
        const float *__restrict__ rstd, T *__restrict__ dx, float *__restrict__ partial, int64_t ldp, int64_t M,
        int32_t N, int32_t nvec) {
    using E = Elem<T>;
    using WV = WeightVec<T, TW>;
    constexpr int EPV = E::kPerVec;
    constexpr bool kRowIsWG = LPR == 0;
    constexpr int RPW = kRowIsWG ? 1 : WG / LPR;
    static_assert(kRowIsWG || WG % LPR == 0, "workgroup must hold whole row groups");
    static_assert(!kRowIsWG || VPT == 1, "a workgroup-sized row holds one vector per lane");
    __shared__ float slots[LPR > 64 || kRowIsWG ? 2 * (WG / 64) : 1];
    __shared__ float comb[RPW > 1 ? WG * EPV : 1];

    const int lpr = kRowIsWG ? (int)blockDim.x : LPR;
    const int lane = kRowIsWG ? (int)threadIdx.x : (int)threadIdx.x % LPR;
    const int grp = kRowIsWG ? 0 : (int)threadIdx.x / LPR;
    const float n = (float)N;
    const uint32_t row_bytes = (uint32_t)nvec * 16u;

    // Byte offset of each of this lane's vectors inside a row block; vectors
    // past the row end get an out-of-range offset (load 0, store nothing).
    uint32_t off[VPT];
    const Buf wb(w, row_bytes * WV::kVecs);
    WV wv[VPT];
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int idx = v * lpr + lane;
        const bool in = idx < nvec;
        off[v] = in ? (uint32_t)grp * row_bytes + (uint32_t)idx * 16u : kOff;
        wv[v].load(wb, idx, in);
    }
    constexpr bool kDwF64 = bwd_vec_dw_f64<T, TW, RES, VPT, WG, PF>();
    DwSums<VPT * EPV, kDwF64> acc;  // sum v * EPV + k: element k of the lane's vector v
    acc.init();

    // rows of the block starting at b that exist (0 past the end)
    auto rows_at = [&](int64_t b) -> uint32_t {
        const int64_t left = M - b;
        return left <= 0 ? 0u : (left < RPW ? (uint32_t)left : (uint32_t)RPW);
    };
    // the block's x, dy (and dh) vectors and its rows' rstd; rows past M read
    // r = 0 and zeros, so they add nothing to dW
    auto load_block = [&](int64_t b, u32x4 (&xo)[VPT], u32x4 (&go)[VPT], u32x4 (&ho)[VPT], float &ro) {
        const int64_t bb = b < M ? b : 0;
        const uint32_t rows = rows_at(b);
        const Buf xb(x + bb * N, rows * row_bytes), gb(dy + bb * N, rows * row_bytes), rb(rstd + bb, rows * 4u);
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            xo[v] = xb.load16<RMSN_BWD_LOAD_AUX>(off[v]);
            go[v] = gb.load16<RMSN_BWD_LOAD_AUX>(off[v]);
        }
        if constexpr (RES) {
            const Buf hb(dh + bb * N, rows * row_bytes);
#pragma unroll
            for (int v = 0; v < VPT; ++v) ho[v] = hb.load16<RMSN_BWD_LOAD_AUX>(off[v]);
        }
        ro = rb.load4((uint32_t)grp * 4u);
    };

    int parity = 0;
    const int64_t step = (int64_t)gridDim.x * RPW;
    int64_t base = (int64_t)blockIdx.x * RPW;

    // dx and the dW sums of the block at `base`, from its loaded vectors
    auto compute = [&](int64_t base, u32x4 (&xv)[VPT], u32x4 (&gv)[VPT], u32x4 (&hv)[VPT], float r) {
        const uint32_t rows = rows_at(base);
        const Buf db(dx + base * N, rows * row_bytes);
        float s = 0.f;
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            float fx[EPV], fg[EPV], fw[EPV];
            E::unpack(xv[v], fx);
            E::unpack(gv[v], fg);
            wv[v].unpack(fw);
#pragma unroll
            for (int k = 0; k < EPV; ++k) {
                s = __builtin_fmaf(fg[k] * fw[k], fx[k], s);
                if constexpr (!kDwF64) acc.add(v * EPV + k, fg[k] * fx[k], r);
            }
        }
        if constexpr (kRowIsWG)
            s = wg_sum<WG>(s, slots, parity);
        else
            s = row_sum<LPR, WG>(s, slots, parity);
        parity ^= 1;
        const float c = r * (r * (r * (s / n)));  // r^3 S/N without forming r^3 (underflows for rows near 1e15)
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            keep_packed(xv[v]);
            keep_packed(gv[v]);
            wv[v].keep();
        }
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            float fx[EPV], fg[EPV], fw[EPV], o[EPV];
            E::unpack(xv[v], fx);
            E::unpack(gv[v], fg);
            wv[v].unpack(fw);
#pragma unroll
            for (int k = 0; k < EPV; ++k) o[k] = __builtin_fmaf(-fx[k], c, r * (fg[k] * fw[k]));
            if constexpr (RES) {
                float fh[EPV];
                E::unpack(hv[v], fh);
#pragma unroll
                for (int k = 0; k < EPV; ++k) o[k] += fh[k];
            }
            db.store16<RMSN_BWD_STORE_AUX>(off[v], E::pack(o));
            // fp64 totals: the dW terms after the store, off the path to the row sum
            if constexpr (kDwF64) {
#pragma unroll
                for (int k = 0; k < EPV; ++k) acc.add(v * EPV + k, fg[k] * fx[k], r);
            }
        }
        acc.end_row();
    };
    auto copy = [&](u32x4 (&xo)[VPT], u32x4 (&go)[VPT], u32x4 (&ho)[VPT], const u32x4 (&xi)[VPT],
                    const u32x4 (&gi)[VPT], const u32x4 (&hi)[VPT]) {
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            xo[v] = xi[v];
            go[v] = gi[v];
            if constexpr (RES) ho[v] = hi[v];
        }
    };
    auto pin_w = [&]() {
#pragma unroll
        for (int v = 0; v < VPT; ++v) wv[v].keep();
    };

    u32x4 xv[VPT], gv[VPT], hv[VPT];  // the block being computed
    float r;
    if constexpr (PF == 0) {
        for (; base < M; base += step) {
            pin_w();
            load_block(base, xv, gv, hv, r);
            compute(base, xv, gv, hv, r);
        }
    } else if constexpr (PF == 1) {
        u32x4 xa[VPT], ga[VPT], ha[VPT];  // the next block
        float ra;
        load_block(base, xa, ga, ha, ra);
        for (; base < M; base += step) {
            pin_w();
            copy(xv, gv, hv, xa, ga, ha);
            r = ra;
            load_block(base + step, xa, ga, ha, ra);
            compute(base, xv, gv, hv, r);
        }
    } else {
        static_assert(PF == 2, "prefetch depth 0, 1 or 2");
        u32x4 xa[VPT], ga[VPT], ha[VPT], xb[VPT], gb[VPT], hb[VPT];  // the next two blocks
        float ra, rb;
        load_block(base, xa, ga, ha, ra);
        load_block(base + step, xb, gb, hb, rb);
        for (; base < M; base += 2 * step) {
            pin_w();
            copy(xv, gv, hv, xa, ga, ha);
            r = ra;
            load_block(base + 2 * step, xa, ga, ha, ra);
            compute(base, xv, gv, hv, r);
            if (base + step >= M) break;
            pin_w();
            copy(xv, gv, hv, xb, gb, hb);
            r = rb;
            load_block(base + 3 * step, xb, gb, hb, rb);
            compute(base + step, xv, gv, hv, r);
        }
    }

    acc.fold();
    float *prow = partial + (int64_t)blockIdx.x * ldp;
    if constexpr (RPW == 1) {
        const Buf pb(prow, (uint32_t)nvec * (uint32_t)(EPV * 4));
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            const int idx = v * lpr + lane;
            if (idx < nvec) {
#pragma unroll
                for (int q = 0; q < EPV / 4; ++q) {
                    u32x4 o;
                    o.x = as_u32(acc.get(v * EPV + 4 * q));
                    o.y = as_u32(acc.get(v * EPV + 4 * q + 1));
                    o.z = as_u32(acc.get(v * EPV + 4 * q + 2));
                    o.w = as_u32(acc.get(v * EPV + 4 * q + 3));
                    pb.store16<RMSN_BWD_PARTIAL_AUX>((uint32_t)(idx * EPV + 4 * q) * 4u, o);
                }
            }
        }
    } else {
        // Add the RPW row groups in group order, one vector slot at a time.
        constexpr int kSlotCols = LPR * EPV;  // columns covered by one vector slot
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            float4 *mine = reinterpret_cast<float4 *>(comb + threadIdx.x * EPV);
#pragma unroll
            for (int q = 0; q < EPV / 4; ++q)
                mine[q] = make_float4(acc.get(v * EPV + 4 * q), acc.get(v * EPV + 4 * q + 1),
                                      acc.get(v * EPV + 4 * q + 2), acc.get(v * EPV + 4 * q + 3));
            __syncthreads();
            for (int q = threadIdx.x; q < kSlotCols; q += WG) {
                const int col = v * kSlotCols + q;
                if (col < N) {
                    double t = comb[q];
#pragma unroll
                    for (int g = 1; g < RPW; ++g) t += comb[g * kSlotCols + q];
                    prow[col] = (float)t;
                }
            }
            __syncthreads();
        }
    }
}

// Wide rows (more than 1024 16-byte vectors): 1024 lanes per row, VPT vectors
// per lane, and each lane's running dW sums kept in LDS instead of registers.
// The sums are per lane (a lane touches only its own slots, laid out so the
// lanes of a wavefront hit consecutive 16-byte words), so they need no
// barrier; moving them out of the register file leaves room for the
// prefetched next row, or, for fp32 rows of up to 32768, for eight vectors
// per lane. Weights stay in registers when they take at most 6 vectors per
// lane counting the prefetch buffers' share (no kernel spills at 6; keeping
// them measured 1.5-2.8% faster than at 4 for bf16 24576 and fp32 20480-24576
// columns; 16-bit rows of 4 vectors with prefetch would spill), and are
// re-read (from cache) at each use otherwise. With RES the residual gradient dh is loaded in the
// second pass, one vector at a time, where it is needed.
#ifndef RMSN_WIDE_KEEP_W_SHARE
#define RMSN_WIDE_KEEP_W_SHARE 6  // weight vectors per lane, counting the prefetch buffers' share
#endif
template <typename T, typename TW, int VPT, bool PF>
constexpr bool wide_keeps_w() {
    return VPT * WeightVec<T, TW>::kVecs * (PF ? 2 : 1) <= RMSN_WIDE_KEEP_W_SHARE;
}

template <typename T, typename TW, bool RES, int VPT, bool PF>
__global__ void __launch_bounds__(kWideLanes) __attribute__((amdgpu_waves_per_eu(kWideLanes / 256)))
bwd_wide(const T *__restrict__ x, const TW *__restrict__ w, const T *__restrict__ dy, const T *__restrict__ dh,
         const float *__restrict__ rstd, T *__restrict__ dx, float *__restrict__ partial, int64_t ldp, int64_t M,
         int32_t N, int32_t nvec) {
    using E = Elem<T>;
    using WV = WeightVec<T, TW>;
    constexpr int LPR = kWideLanes;
    constexpr int EPV = E::kPerVec;
    constexpr int Q = EPV / 4;  // float4 words of dW sums per vector
    constexpr bool kKeepW = wide_keeps_w<T, TW, VPT, PF>();
    static_assert(VPT * EPV * LPR * 4 <= kWideLdsBytes, "dW sums must fit in LDS");
    __shared__ float slots[2 * (LPR / 64)];
    __shared__ float4 acc[VPT * Q * LPR];

    const int lane = threadIdx.x;
    const float n = (float)N;
    const uint32_t row_bytes = (uint32_t)nvec * 16u;
    const Buf wb(w, row_bytes * WV::kVecs);

    uint32_t off[VPT];
    WV wv[kKeepW ? VPT : 1];
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int idx = v * LPR + lane;
        off[v] = idx < nvec ? (uint32_t)idx * 16u : kOff;
        if constexpr (kKeepW) wv[v].load(wb, idx, idx < nvec);
#pragma unroll
        for (int q = 0; q < Q; ++q) acc[(v * Q + q) * LPR + lane] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    // weights of vector slot v: the kept registers, or a (cached) reload
    auto weights = [&](int v, float (&fw)[EPV]) {
        if constexpr (kKeepW) {
            wv[v].unpack(fw);
        } else {
            WV t;
            t.load(wb, v * LPR + lane, off[v] != kOff);
            t.unpack(fw);
        }
    };
    auto load_block = [&](int64_t b, u32x4 (&xo)[VPT], u32x4 (&go)[VPT], float &ro) {
        const int64_t bb = b < M ? b : 0;
        const uint32_t bytes = b < M ? row_bytes : 0u;
        const Buf xb(x + bb * N, bytes), gb(dy + bb * N, bytes), rb(rstd + bb, b < M ? 4u : 0u);
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            xo[v] = xb.load16<RMSN_BWD_LOAD_AUX>(off[v]);
            go[v] = gb.load16<RMSN_BWD_LOAD_AUX>(off[v]);
        }
        ro = rb.load4(0u);
    };

    int parity = 0;
    const int64_t step = (int64_t)gridDim.x;
    int64_t row = (int64_t)blockIdx.x;
    u32x4 xn[VPT], gn[VPT];
    float rn = 0.f;
    if constexpr (PF) load_block(row, xn, gn, rn);
    for (; row < M; row += step) {
        if constexpr (kKeepW) {
#pragma unroll
            for (int v = 0; v < VPT; ++v) wv[v].keep();
        }
        u32x4 xv[VPT], gv[VPT];
        float r;
        if constexpr (PF) {
#pragma unroll
            for (int v = 0; v < VPT; ++v) {
                xv[v] = xn[v];
                gv[v] = gn[v];
            }
            r = rn;
            load_block(row + step, xn, gn, rn);
        } else {
            load_block(row, xv, gv, r);
        }

        float s = 0.f;
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            float fx[EPV], fg[EPV], fw[EPV];
            E::unpack(xv[v], fx);
            E::unpack(gv[v], fg);
            weights(v, fw);
#pragma unroll
            for (int k = 0; k < EPV; ++k) s = __builtin_fmaf(fg[k] * fw[k], fx[k], s);
        }
        s = row_sum<LPR, LPR>(s, slots, parity);
        parity ^= 1;
        const float c = r * (r * (r * (s / n)));
        const Buf db(dx + row * N, row_bytes);
        const Buf hb(RES ? dh + row * N : dx, RES ? row_bytes : 0u);
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            keep_packed(xv[v]);
            keep_packed(gv[v]);
        }
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            float fx[EPV], fg[EPV], fw[EPV], o[EPV];
            E::unpack(xv[v], fx);
            E::unpack(gv[v], fg);
            weights(v, fw);
#pragma unroll
            for (int k = 0; k < EPV; ++k) o[k] = __builtin_fmaf(-fx[k], c, r * (fg[k] * fw[k]));
            if constexpr (RES) {
                float fh[EPV];
                E::unpack(hb.load16<RMSN_BWD_LOAD_AUX>(off[v]), fh);
#pragma unroll
                for (int k = 0; k < EPV; ++k) o[k] += fh[k];
            }
            db.store16<RMSN_BWD_STORE_AUX>(off[v], E::pack(o));
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                float4 &a = acc[(v * Q + q) * LPR + lane];
                a.x = __builtin_fmaf(fg[4 * q] * fx[4 * q], r, a.x);
                a.y = __builtin_fmaf(fg[4 * q + 1] * fx[4 * q + 1], r, a.y);
                a.z = __builtin_fmaf(fg[4 * q + 2] * fx[4 * q + 2], r, a.z);
                a.w = __builtin_fmaf(fg[4 * q + 3] * fx[4 * q + 3], r, a.w);
            }
        }
    }

    const Buf pb(partial + (int64_t)blockIdx.x * ldp, (uint32_t)nvec * (uint32_t)(EPV * 4));
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int idx = v * LPR + lane;
        if (idx < nvec) {
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const float4 a = acc[(v * Q + q) * LPR + lane];
                u32x4 o;
                o.x = as_u32(a.x);
                o.y = as_u32(a.y);
                o.z = as_u32(a.z);
                o.w = as_u32(a.w);
                pb.store16<RMSN_BWD_PARTIAL_AUX>((uint32_t)(idx * EPV + 4 * q) * 4u, o);
            }
        }
    }
}

// Scalar backward (any N, any alignment): one workgroup per row at a time,
// element loads. Each lane owns columns threadIdx.x + k*kScalarWG of the
// workgroup's dW running sums for the whole kernel (no lane touches another's,
// so no barrier), kept in LDS when the row has at most kScalarLdsCols columns
// (LDS) and in the workgroup's partial row in memory otherwise; the partial
// row is written once at the end in the LDS case. The sums see the same fma
// sequence either way, so dW has the same bits.
template <typename T, typename TW, bool RES, bool LDS>
__global__ void __launch_bounds__(kScalarWG)
bwd_scalar(const T *__restrict__ x, const TW *__restrict__ w, const T *__restrict__ dy, const T *__restrict__ dh,
           const float *__restrict__ rstd, T *__restrict__ dx, float *__restrict__ partial, int64_t ldp, int64_t M,
           int32_t N, int32_t /*nvec*/) {
    using E = Elem<T>;
    __shared__ float slots[2 * (kScalarWG / 64)];
    __shared__ float sums[LDS ? kScalarLdsCols : 1];
    const float n = (float)N;
    float *prow = partial + (int64_t)blockIdx.x * ldp;
    float *acc = LDS ? sums : prow;
    for (int j = threadIdx.x; j < N; j += kScalarWG) acc[j] = 0.f;
    int parity = 0;
    for (int64_t row = blockIdx.x; row < M; row += gridDim.x) {
        const int64_t o = row * (int64_t)N;
        const float r = rstd[row];
        float s = 0.f;
        for (int j = threadIdx.x; j < N; j += kScalarWG)
            s = __builtin_fmaf(E::load(dy + o + j) * Elem<TW>::load(w + j), E::load(x + o + j), s);
        s = row_sum<kScalarWG, kScalarWG>(s, slots, parity);
        parity ^= 1;
        const float c = r * (r * (r * (s / n)));
        for (int j = threadIdx.x; j < N; j += kScalarWG) {
            const float fx = E::load(x + o + j), fg = E::load(dy + o + j), fw = Elem<TW>::load(w + j);
            float g = __builtin_fmaf(-fx, c, r * (fg * fw));
            if constexpr (RES) g += E::load(dh + o + j);
            E::store(dx + o + j, g);
            acc[j] = __builtin_fmaf(fg * fx, r, acc[j]);
        }
    }
    if constexpr (LDS) {
        for (int j = threadIdx.x; j < N; j += kScalarWG) prow[j] = acc[j];
    }
}

}  // namespace rmsn
