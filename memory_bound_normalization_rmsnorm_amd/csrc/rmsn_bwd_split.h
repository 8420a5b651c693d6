// rmsn_bwd_split.h -- backward for rows wider than one workgroup's dW sums:
// each row split over K workgroups that exchange their partial row sums.
//
// The wide-row kernel (bwd_wide) keeps a workgroup's dW running sums for the
// whole row in LDS, 4 bytes per column: at most 32768 columns in 128 KiB.
// Wider rows are split into K column slices of at most that many columns
// (the Quack study, "What a tuned RMSNorm kernel actually costs on Hopper",
// section 03, spreads its widest rows over a cluster of CTAs; AMD has no
// clusters, so the workgroups of a row meet through global memory). Group g
// of K consecutive workgroups walks rows g, g + G, ... (G = grid / K), member
// k owning slice k: it loads its slice of x and dy once, computes its part of
// S = sum_j (dy_j w_j) x_j, publishes that part, waits for the other K - 1
// parts, adds all K in member order (so every member gets the same bits), and
// finishes dx and its dW sums for the slice. The group's K slices of dW sums
// make one partial row; the fixed-order combine adds the G partial rows. No
// atomic read-modify-write anywhere: each member writes only its own slot.
//
// Exchange: member k of group g owns slot g * K + k, two 64-bit words. For
// its i-th row it stores, in one relaxed atomic store at device scope, the
// word (i + 1) << 32 | bits(part) into word[i & 1]; readers poll their
// partners' word[i & 1] with relaxed atomic loads at device scope (one lane
// per partner, all partners in each polling round) until the high half reads
// i + 1, and take the low half. Tag and value travel in one
// word, so no fence orders them, and device-scope accesses are coherent
// across the XCDs' separate L2 caches. Two words suffice: a member reaches
// its row i + 2 only after every partner published row i + 1, which each
// does after reading row i. The host zeroes the slots before each launch (a
// fill kernel, not a memset, so the call can be captured in a graph), so no
// tag of an earlier launch is mistaken for this one's. The grid is at most
// what stays resident, so every partner runs; the wait is still bounded: a
// member that gives up uses a NaN sum for that row and every later one, so a
// grid that cannot be co-resident gives NaN outputs instead of a hang.
#pragma once

#include "rmsn_device.h"
#include "rmsn_tables.h"

namespace rmsn {

// One member's exchange slot: 16 bytes.
struct SplitSlot {
    uint64_t word[2];
};

// Polling rounds over a member's whole walk before it gives up (each round a
// device-scope load per partner not yet seen and a short sleep, about a
// microsecond): about a second in all, far beyond any real wait
// (microseconds).
constexpr uint32_t kSplitSpinLimit = 1u << 20;

// Weight vectors per lane kept in registers at two workgroups per CU. Keeping
// the two of a 16-bit row costs a 12-16 byte spill at 64 VGPRs, and still
// measured 5-7% faster than re-reading them from cache each row without the
// spill (bf16 4096 x 65536: 297.3 against 318.0 us; 1024 x 262144: 387.1
// against 411.0; the residual backward 373.3 against 391.3).
#ifndef RMSN_SPLIT_KEEP_W_TWO
#define RMSN_SPLIT_KEEP_W_TWO 2
#endif

// Waves per SIMD a member asks for: two workgroups per CU (64 VGPRs each)
// when its dW sums take at most 64 KiB of LDS (2 vectors of 8 16-bit
// elements per lane, or 4 of 4 fp32), one above.
constexpr int split_waves_per_eu(int vpt, int epv) { return (vpt * epv <= 16 ? 2 : 1) * kWideLanes / 256; }

template <typename T, typename TW, bool RES, int VPT, bool PF>
__global__ void __launch_bounds__(kWideLanes) __attribute__((amdgpu_waves_per_eu(split_waves_per_eu(VPT, Elem<T>::kPerVec))))
bwd_split(const T *__restrict__ x, const TW *__restrict__ w, const T *__restrict__ dy, const T *__restrict__ dh,
          const float *__restrict__ rstd, T *__restrict__ dx, float *__restrict__ partial, int64_t ldp, int64_t M,
          int32_t N, int32_t nvec, int32_t K, SplitSlot *__restrict__ xch) {
    using E = Elem<T>;
    using WV = WeightVec<T, TW>;
    constexpr int LPR = kWideLanes;
    constexpr int EPV = E::kPerVec;
    constexpr int Q = EPV / 4;  // float4 words of dW sums per vector
    // weights kept in registers as by the wide-row kernel; at two workgroups
    // per CU (64 VGPRs) only up to RMSN_SPLIT_KEEP_W_TWO weight vectors per lane
    constexpr bool kTwoPerCU = split_waves_per_eu(VPT, EPV) > kWideLanes / 256;
    constexpr bool kKeepW =
        wide_keeps_w<T, TW, VPT, PF>() && (!kTwoPerCU || VPT * WV::kVecs <= RMSN_SPLIT_KEEP_W_TWO);
    static_assert(VPT * EPV * LPR * 4 <= kWideLdsBytes, "dW sums must fit in LDS");
    __shared__ float slots[2 * (LPR / 64)];
    __shared__ float total[2];
    __shared__ float4 acc[VPT * Q * LPR];

    const int lane = threadIdx.x;
    const int k = (int)(blockIdx.x % (uint32_t)K);
    const int64_t g = (int64_t)(blockIdx.x / (uint32_t)K);
    const int64_t G = (int64_t)(gridDim.x / (uint32_t)K);
    const float n = (float)N;
    const uint32_t row_bytes = (uint32_t)nvec * 16u;
    const int slice = (nvec + K - 1) / K;  // vectors per slice
    const int v0 = k * slice;
    const int v1 = v0 + slice < nvec ? v0 + slice : nvec;
    const Buf wb(w, row_bytes * WV::kVecs);

    uint32_t off[VPT];
    WV wv[kKeepW ? VPT : 1];
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int idx = v0 + v * LPR + lane;
        off[v] = idx < v1 ? (uint32_t)idx * 16u : kOff;
        if constexpr (kKeepW) wv[v].load(wb, idx, idx < v1);
#pragma unroll
        for (int q = 0; q < Q; ++q) acc[(v * Q + q) * LPR + lane] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    auto weights = [&](int v, float (&fw)[EPV]) {
        if constexpr (kKeepW) {
            wv[v].unpack(fw);
        } else {
            WV t;
            const int idx = v0 + v * LPR + lane;
            t.load(wb, idx, off[v] != kOff);
            t.unpack(fw);
        }
    };
    auto load_row = [&](int64_t b, u32x4 (&xo)[VPT], u32x4 (&go)[VPT], float &ro) {
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

    SplitSlot *const mine = xch + g * K + k;
    SplitSlot *const group = xch + g * K;
    int parity = 0;
    uint32_t it = 0;
    uint32_t spins = 0;  // polling rounds so far (wavefront 0) over the whole walk; at the limit every later sum is NaN
    int64_t row = g;
    u32x4 xn[VPT], gn[VPT];
    float rn = 0.f;
    if constexpr (PF) load_row(row, xn, gn, rn);
    for (; row < M; row += G, ++it) {
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
            load_row(row + G, xn, gn, rn);
        } else {
            load_row(row, xv, gv, r);
        }

        float s = 0.f;
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            float fx[EPV], fg[EPV], fw[EPV];
            E::unpack(xv[v], fx);
            E::unpack(gv[v], fg);
            weights(v, fw);
#pragma unroll
            for (int e = 0; e < EPV; ++e) s = __builtin_fmaf(fg[e] * fw[e], fx[e], s);
        }
        s = row_sum<LPR, LPR>(s, slots, parity);
        parity ^= 1;
        // Publish this slice's part, wait for the others, add all K in member
        // order. Wavefront 0 does it: lane p < K polls member p's word, all
        // partners at once, until every tag reads this row's; the K parts are
        // then added in member order and handed to the workgroup.
        if (lane < 64) {
            const uint64_t tag = (uint64_t)(it + 1u) << 32;
            if (lane == 0)
                __hip_atomic_store(&mine->word[it & 1u], tag | as_u32(s), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            bool ready = lane >= K || lane == k;
            float part = s;
            while (spins < kSplitSpinLimit) {
                if (!ready) {
                    const uint64_t v =
                        __hip_atomic_load(&group[lane].word[it & 1u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if ((v & ~uint64_t(0xffffffffu)) == tag) {
                        ready = true;
                        part = __uint_as_float((uint32_t)v);
                    }
                }
                if (__all(ready)) break;
                ++spins;
                __builtin_amdgcn_s_sleep(2);
            }
            if (!ready) part = __builtin_nanf("");
            float t = 0.f;
            for (int p = 0; p < K; ++p) t += __shfl(part, p);
            if (lane == 0) total[it & 1u] = t;
        }
        __syncthreads();
        const float S = total[it & 1u];
        const float c = r * (r * (r * (S / n)));
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
            for (int e = 0; e < EPV; ++e) o[e] = __builtin_fmaf(-fx[e], c, r * (fg[e] * fw[e]));
            if constexpr (RES) {
                float fh[EPV];
                E::unpack(hb.load16<RMSN_BWD_LOAD_AUX>(off[v]), fh);
#pragma unroll
                for (int e = 0; e < EPV; ++e) o[e] += fh[e];
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

    // this slice of the group's partial row
    const Buf pb(partial + g * ldp, (uint32_t)nvec * (uint32_t)(EPV * 4));
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int idx = v0 + v * LPR + lane;
        if (idx < v1) {
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

}  // namespace rmsn
