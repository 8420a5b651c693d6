// rmsn_bwd_lds.h -- backward row kernel with the row blocks staged through
// LDS by gfx950's 16-byte global->LDS copies, ST blocks in flight.
//
// The same arithmetic and the same fixed row -> workgroup map as bwd_vec
// (rmsn_bwd_kernels.h): per row i, with r = rstd_i and V_ij = dy_ij * w_j,
//     dx_ij = r V_ij - x_ij r^3 (sum_j V_ij x_ij) / N,   dW partial += dy_ij x_ij r
// ("RMSNorm backward (almost) without the column reduction", sections "The
// backward pass" and "The persistent kernel"). What differs is how the next
// row blocks arrive. The persistent page pipelines its loads through shared
// memory with asynchronous copies, and the Quack study ("What a tuned RMSNorm
// kernel actually costs on Hopper", sections 06 and 09) found the copy path
// and the depth of that pipeline to be the constants that mattered most for
// its backward. Here a ring of ST LDS stages holds the x, dy (and dh) vectors
// and the rstd of ST row blocks: buffer_load_dwordx4 ... lds writes each
// lane's 16 bytes straight into the lane's own LDS slot, without passing
// through VGPRs, so the depth is bounded by LDS (160 KiB per CU) and not by
// registers (the register ring of bwd_vec holds at most two blocks).
//
// Ordering. Every lane reads back only the slot its own copy wrote, and
// rstd is copied once per wavefront into that wavefront's own slots, so no
// stage needs a barrier: a wavefront waits for its own copies with
// s_waitcnt vmcnt. Vector memory operations of a wavefront complete in issue
// order, so "stage j has landed" is "at most K newer operations are
// outstanding": the prologue issues ST groups of L copies, and iteration j
// then waits, reads stage j % ST, refills it with block j + ST (L copies)
// and stores one dx vector, so K = (ST - 1) * L + min(j, ST). The LDS reads
// are inline asm (with their own lgkmcnt wait), because the compiler guards
// any LDS read that may alias an outstanding global->LDS copy with
// vmcnt(0), which would drain the whole ring each row; for the same reason
// the cross-wavefront row sum uses a bare s_barrier after lgkmcnt(0) rather
// than __syncthreads, whose release fence also waits for vmcnt(0). The ring
// refill of a stage is issued after the lane's own reads of it completed, so
// a slot is never overwritten while it is read.
//
// Rows past M and vectors past the row end are read through buffer
// resources whose record counts exclude them; their values are zeroed in
// registers after the read whatever the copy left in LDS, so they add
// nothing. Before the partial dW row is written (and before the workgroup
// ends) every copy has completed.
#pragma once

#include "rmsn_device.h"
#include "rmsn_tables.h"

namespace rmsn {

typedef __attribute__((address_space(3))) void lds_void;

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_off(const void *p) {
    return (uint32_t)(uintptr_t)(const lds_void *)p;
}

// rstd floats a wavefront copies per stage: one per lane (lanes past the
// block's rows read past the buffer's record count), so the copy needs no
// branch; at most this many rows per workgroup.
constexpr int kLdsRstdSlots = 64;

// Bytes of LDS the stage ring takes: per stage NIN 16-byte vectors per lane
// and kLdsRstdSlots rstd floats per wavefront.
constexpr int lds_ring_bytes(int st, int nin, int wg) { return st * (nin * wg * 16 + (wg / 64) * kLdsRstdSlots * 4); }

// s_waitcnt vmcnt(BASE + m * Q) for the runtime m in [0, M] (m is wave-uniform).
template <int BASE, int M, int Q = 1>
__device__ __forceinline__ void wait_vm(int m) {
    if constexpr (M == 0) {
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(BASE) : "memory");
    } else {
        if (m >= M) {
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(BASE + M * Q) : "memory");
            return;
        }
        wait_vm<BASE, M - 1, Q>(m);
    }
}

// A workgroup barrier that waits only for LDS operations (lgkmcnt), not for
// outstanding global->LDS copies of later stages.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// row_sum (rmsn_device.h) with lds_barrier in place of __syncthreads.
template <int LPR, int WG>
__device__ __forceinline__ float row_sum_nf(float v, float *slots, int parity) {
    if constexpr (LPR <= 64) {
        return group_sum<LPR>(v);
    } else {
        constexpr int kWaves = WG / 64;
        constexpr int kWavesPerRow = LPR / 64;
        v = group_sum<64>(v);
        const int wave = threadIdx.x >> 6;
        float *buf = slots + parity * kWaves;
        if ((threadIdx.x & 63) == 0) buf[wave] = v;
        lds_barrier();
        const int first = wave - (wave % kWavesPerRow);
        float s = buf[first];
#pragma unroll
        for (int k = 1; k < kWavesPerRow; ++k) s += buf[first + k];
        return s;
    }
}

// wg_sum (rmsn_device.h) with lds_barrier in place of __syncthreads.
template <int WG>
__device__ __forceinline__ float wg_sum_nf(float v, float *slots, int parity) {
    v = group_sum<64>(v);
    const int waves = (int)(blockDim.x >> 6);
    float *buf = slots + parity * (WG / 64);
    if ((threadIdx.x & 63) == 0) buf[threadIdx.x >> 6] = v;
    lds_barrier();
    float s = buf[0];
    for (int k = 1; k < waves; ++k) s += buf[k];
    return s;
}

// The lane's stage vectors (x at `a`, dy at a + STRIDE, dh at a + 2 STRIDE)
// and its row's rstd (at `ar`), read and waited for in one asm block (the
// outputs are early-clobber, so no destination overlaps an address).
template <bool RES, int STRIDE>
__device__ __forceinline__ void lds_read_stage(uint32_t a, uint32_t ar, u32x4 &x, u32x4 &g, u32x4 &h, float &r) {
    if constexpr (RES) {
        asm volatile(
            "ds_read_b128 %0, %4\n\t"
            "ds_read_b128 %1, %4 offset:%6\n\t"
            "ds_read_b128 %2, %4 offset:%7\n\t"
            "ds_read_b32 %3, %5\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(x), "=&v"(g), "=&v"(h), "=&v"(r)
            : "v"(a), "v"(ar), "n"(STRIDE), "n"(2 * STRIDE)
            : "memory");
    } else {
        asm volatile(
            "ds_read_b128 %0, %3\n\t"
            "ds_read_b128 %1, %3 offset:%5\n\t"
            "ds_read_b32 %2, %4\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(x), "=&v"(g), "=&v"(r)
            : "v"(a), "v"(ar), "n"(STRIDE)
            : "memory");
    }
}

// The lane's weight vector(s) (KV of them, STRIDE bytes apart), read and
// waited for in one asm block.
template <int KV, int STRIDE>
__device__ __forceinline__ void lds_read_weights(uint32_t a, u32x4 (&v)[KV]) {
    if constexpr (KV == 1) {
        asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v[0]) : "v"(a) : "memory");
    } else {
        static_assert(KV == 2, "one or two weight vectors per activation vector");
        asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:%3\n\ts_waitcnt lgkmcnt(0)"
                     : "=&v"(v[0]), "=&v"(v[1])
                     : "v"(a), "n"(STRIDE)
                     : "memory");
    }
}

// LPR lanes per row (64..1024, a power of two), or 0: the row is the whole
// workgroup, its size (a multiple of 64 up to WG) set at launch. One 16-byte
// vector per lane. ST: stages (row blocks in flight), 2..8.
template <typename T, typename TW, bool RES, int LPR, int WG, int ST>
__global__ void __launch_bounds__(WG) __attribute__((amdgpu_waves_per_eu(WG / 256 > 1 ? WG / 256 : 1)))
bwd_lds(const T *__restrict__ x, const TW *__restrict__ w, const T *__restrict__ dy, const T *__restrict__ dh,
        const float *__restrict__ rstd, T *__restrict__ dx, float *__restrict__ partial, int64_t ldp, int64_t M,
        int32_t N, int32_t nvec) {
    using E = Elem<T>;
    using WV = WeightVec<T, TW>;
    constexpr int EPV = E::kPerVec;
    constexpr bool kRowIsWG = LPR == 0;
    constexpr int RPW = kRowIsWG ? 1 : WG / LPR;
    constexpr int NIN = RES ? 3 : 2;
    constexpr int L = NIN + 1;  // copies per stage and lane: the inputs and rstd
    constexpr int kWaves = WG / 64;
    constexpr int kStride = WG * 16;  // bytes between a stage's x, dy and dh vectors
    static_assert(kRowIsWG || (LPR >= 64 && WG % LPR == 0), "rows of whole wavefronts");
    static_assert(RPW <= kLdsRstdSlots, "rstd slots per wavefront");
    static_assert(ST >= 2 && ST <= 8 && (ST - 1) * L + ST <= 63, "vmcnt range");
    static_assert(WV::kVecs <= NIN, "the weights borrow the last stage's input slots");
    static_assert(lds_ring_bytes(ST, NIN, WG) + 2 * kWaves * 4 <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(16))) u32x4 ring[ST * NIN * WG];
    __shared__ float rst[ST * kWaves * kLdsRstdSlots];
    __shared__ float slots[2 * kWaves];

    const int lane = kRowIsWG ? (int)threadIdx.x : (int)threadIdx.x % LPR;
    const int grp = kRowIsWG ? 0 : (int)threadIdx.x / LPR;
    const int wave = (int)threadIdx.x >> 6;
    const int wlane = (int)threadIdx.x & 63;
    const float n = (float)N;
    const uint32_t row_bytes = (uint32_t)nvec * 16u;
    const bool vin = lane < nvec;
    const uint32_t off = vin ? (uint32_t)grp * row_bytes + (uint32_t)lane * 16u : kOff;

    DwSums<EPV, true> acc;  // one workgroup per CU: the fp64 totals cost no residency
    acc.init();

    const int64_t step = (int64_t)gridDim.x * RPW;
    int64_t base = (int64_t)blockIdx.x * RPW;
    auto rows_at = [&](int64_t b) -> uint32_t {
        const int64_t left = M - b;
        return left <= 0 ? 0u : (left < RPW ? (uint32_t)left : (uint32_t)RPW);
    };
    // Copies of the block at b into stage s: this lane's x, dy (dh) vectors,
    // and rstd of row b + (lane in wavefront), within the block's rows.
    auto issue = [&](int64_t b, int s) {
        const int64_t bb = b < M ? b : 0;
        const uint32_t rows = rows_at(b);
        const __amdgpu_buffer_rsrc_t xr = Buf(x + bb * N, rows * row_bytes).r;
        const __amdgpu_buffer_rsrc_t gr = Buf(dy + bb * N, rows * row_bytes).r;
        u32x4 *st = ring + s * NIN * WG + wave * 64;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void *)st, 16, off, 0, 0, RMSN_BWD_LOAD_AUX);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(gr, (lds_void *)(st + WG), 16, off, 0, 0, RMSN_BWD_LOAD_AUX);
        if constexpr (RES) {
            const __amdgpu_buffer_rsrc_t hr = Buf(dh + bb * N, rows * row_bytes).r;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(hr, (lds_void *)(st + 2 * WG), 16, off, 0, 0,
                                                     RMSN_BWD_LOAD_AUX);
        }
        const __amdgpu_buffer_rsrc_t rr = Buf(rstd + bb, rows * 4u).r;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (lds_void *)(rst + (s * kWaves + wave) * kLdsRstdSlots), 4,
                                                 (uint32_t)wlane * 4u, 0, 0, 0);
        asm volatile("" ::: "memory");  // keep the copies of this stage ahead of later memory operations
    };

    // The weights take the same path, into the lane's own slots of the last
    // stage, ahead of the first ST - 1 stages' copies; once they have landed
    // (the (ST - 1) * L copies after them may still be in flight) they are
    // read into registers and that stage is filled. A register load here
    // would be waited for with vmcnt(0) by the compiler, draining the ring.
    WV wv;
    {
        const __amdgpu_buffer_rsrc_t wr = Buf(w, row_bytes * WV::kVecs).r;
        u32x4 *wst = ring + (ST - 1) * NIN * WG + wave * 64;
#pragma unroll
        for (int q = 0; q < WV::kVecs; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_void *)(wst + q * WG), 16,
                                                     vin ? (uint32_t)(lane * WV::kVecs + q) * 16u : kOff, 0, 0, 0);
        asm volatile("" ::: "memory");
        for (int s = 0; s + 1 < ST; ++s) issue(base + (int64_t)s * step, s);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((ST - 1) * L) : "memory");
        lds_read_weights<WV::kVecs, kStride>(lds_off(wst + wlane), wv.v);
        if (!vin) {
#pragma unroll
            for (int q = 0; q < WV::kVecs; ++q) wv.v[q] = u32x4{0u, 0u, 0u, 0u};
        }
        issue(base + (int64_t)(ST - 1) * step, ST - 1);
    }

    const uint32_t a0 = lds_off(ring + wave * 64 + wlane);
    const uint32_t ar0 = lds_off(rst + wave * kLdsRstdSlots + grp);
    int parity = 0, s = 0, m = 0;
    for (; base < M; base += step) {
        wait_vm<(ST - 1) * L, ST>(m);
        u32x4 xv, gv, hv;
        float r;
        lds_read_stage<RES, kStride>(a0 + (uint32_t)(s * NIN * WG * 16), ar0 + (uint32_t)(s * kWaves * kLdsRstdSlots * 4),
                                     xv, gv, hv, r);
        issue(base + (int64_t)ST * step, s);
        s = s + 1 == ST ? 0 : s + 1;
        m = m < ST ? m + 1 : ST;

        const bool row_ok = base + grp < M;
        const u32x4 z = {0u, 0u, 0u, 0u};
        if (!(row_ok && vin)) {
            xv = z;
            gv = z;
            hv = z;
        }
        if (!row_ok) r = 0.f;

        float sacc = 0.f;
        {
            float fx[EPV], fg[EPV], fw[EPV];
            E::unpack(xv, fx);
            E::unpack(gv, fg);
            wv.unpack(fw);
#pragma unroll
            for (int k = 0; k < EPV; ++k) sacc = __builtin_fmaf(fg[k] * fw[k], fx[k], sacc);
        }
        if constexpr (kRowIsWG)
            sacc = wg_sum_nf<WG>(sacc, slots, parity);
        else
            sacc = row_sum_nf<LPR, WG>(sacc, slots, parity);
        parity ^= 1;
        const float c = r * (r * (r * (sacc / n)));  // r^3 S/N without forming r^3
        keep_packed(xv);
        keep_packed(gv);
        wv.keep();
        float fx[EPV], fg[EPV], fw[EPV], o[EPV];
        E::unpack(xv, fx);
        E::unpack(gv, fg);
        wv.unpack(fw);
#pragma unroll
        for (int k = 0; k < EPV; ++k) o[k] = __builtin_fmaf(-fx[k], c, r * (fg[k] * fw[k]));
        if constexpr (RES) {
            float fh[EPV];
            E::unpack(hv, fh);
#pragma unroll
            for (int k = 0; k < EPV; ++k) o[k] += fh[k];
        }
        const Buf db(dx + base * N, rows_at(base) * row_bytes);
        db.store16<RMSN_BWD_STORE_AUX>(off, E::pack(o));
        // the dW terms after the row's store, off the path to the row sum
#pragma unroll
        for (int k = 0; k < EPV; ++k) acc.add(k, fg[k] * fx[k], r);
        acc.end_row();
    }
    acc.fold();
    // every copy has landed before LDS is reused or the workgroup ends
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    float *prow = partial + (int64_t)blockIdx.x * ldp;
    if constexpr (RPW == 1) {
        if (vin) {
            const Buf pb(prow, (uint32_t)nvec * (uint32_t)(EPV * 4));
#pragma unroll
            for (int q = 0; q < EPV / 4; ++q) {
                u32x4 o;
                o.x = as_u32(acc.get(4 * q));
                o.y = as_u32(acc.get(4 * q + 1));
                o.z = as_u32(acc.get(4 * q + 2));
                o.w = as_u32(acc.get(4 * q + 3));
                pb.store16<RMSN_BWD_PARTIAL_AUX>((uint32_t)(lane * EPV + 4 * q) * 4u, o);
            }
        }
    } else {
        // the RPW row groups added in group order through LDS (the ring is free now)
        __syncthreads();
        float *comb = reinterpret_cast<float *>(ring);
        static_assert(ST * NIN * WG * 16 >= WG * EPV * 4, "combine buffer fits in the ring");
        float4 *mine = reinterpret_cast<float4 *>(comb + threadIdx.x * EPV);
#pragma unroll
        for (int q = 0; q < EPV / 4; ++q)
            mine[q] = make_float4(acc.get(4 * q), acc.get(4 * q + 1), acc.get(4 * q + 2), acc.get(4 * q + 3));
        __syncthreads();
        constexpr int kSlotCols = LPR * EPV;
        for (int q = threadIdx.x; q < kSlotCols; q += WG) {
            if (q < N) {
                double t = comb[q];
#pragma unroll
                for (int g = 1; g < RPW; ++g) t += comb[g * kSlotCols + q];
                prow[q] = (float)t;
            }
        }
    }
}

}  // namespace rmsn

namespace rmsn {

// Wide rows (more than 1024 16-byte vectors: VPT per lane on LPR = 512 or
// 1024 lanes), one row per workgroup at a time, with the next row(s) staged
// through LDS. bwd_wide keeps each lane's dW sums in LDS and re-reads weights
// from cache, because the register file holds the row and its prefetched
// successor. Here the successor lands in LDS instead (ST stages of a whole
// row of x and dy: 128 KiB at 32768 16-bit columns, so one stage; two at
// 16384), which leaves the registers for the dW sums (VPT x 8 floats), and
// for the weights when the lane's register budget allows (512 registers per
// SIMD lane shared by LPR / 256 wavefronts: 128 each at 1024 lanes, 256 at
// 512 lanes; re-read from cache otherwise). Ordering as in bwd_lds: each lane
// reads back only its own slots and waits for its own copies; with Q = VPT dx
// stores per row the wait before row j is vmcnt((ST - 1) * L + min(j, ST) * Q).
template <typename T, typename TW, int LPR, int VPT>
constexpr bool wide_lds_keeps_w() {
    // weight vectors per lane that fit beside the row and the dW sums without
    // spilling (the build's resource report): 2 at 1024 lanes, 6 at 512
    return VPT * WeightVec<T, TW>::kVecs <= (LPR == 1024 ? 2 : 6);
}

template <typename T, typename TW, int LPR, int VPT, int ST>
__global__ void __launch_bounds__(LPR) __attribute__((amdgpu_waves_per_eu(LPR / 256)))
bwd_wide_lds(const T *__restrict__ x, const TW *__restrict__ w, const T *__restrict__ dy,
             const T *__restrict__ dh, const float *__restrict__ rstd, T *__restrict__ dx,
             float *__restrict__ partial, int64_t ldp, int64_t M, int32_t N, int32_t nvec) {
    using E = Elem<T>;
    using WV = WeightVec<T, TW>;
    constexpr int EPV = E::kPerVec;
    constexpr int kWaves = LPR / 64;
    constexpr int L = 2 * VPT + 1;  // copies per stage and lane: x and dy vectors, rstd
    constexpr int Q = VPT;          // dx stores per row and lane
    constexpr bool kKeepW = wide_lds_keeps_w<T, TW, LPR, VPT>();
    constexpr int kVecBytes = LPR * 16;  // bytes between consecutive vector slots of a stage
    static_assert(LPR == 512 || LPR == 1024, "512 or 1024 lanes");
    static_assert(ST >= 1 && (ST - 1) * L + ST * Q <= 63, "vmcnt range");
    static_assert(ST * 2 * VPT * kVecBytes + ST * kWaves * kLdsRstdSlots * 4 + 2 * kWaves * 4 <= 160 * 1024, "LDS");
    // stage s, input t (0 x, 1 dy), vector v: ring[((s * 2 + t) * VPT + v) * LPR + lane]
    __shared__ __attribute__((aligned(16))) u32x4 ring[ST * 2 * VPT * LPR];
    // the rstd copy of wavefront w for stage s: rst[(s * kWaves + w) * kLdsRstdSlots + lane] (lane 0: the row's)
    __shared__ float rst[ST * kWaves * kLdsRstdSlots];
    __shared__ float slots[2 * kWaves];

    const int lane = threadIdx.x;
    const int wave = lane >> 6;
    const float n = (float)N;
    const uint32_t row_bytes = (uint32_t)nvec * 16u;
    const Buf wb(w, row_bytes * WV::kVecs);
    uint32_t off[VPT];
    bool vin[VPT];
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int idx = v * LPR + lane;
        vin[v] = idx < nvec;
        off[v] = vin[v] ? (uint32_t)idx * 16u : kOff;
    }
    // weights of vector slot v: kept registers, or a (cached) reload
    WV wv[kKeepW ? VPT : 1];
    if constexpr (kKeepW) {
#pragma unroll
        for (int v = 0; v < VPT; ++v) wv[v].load(wb, v * LPR + lane, vin[v]);
    }
    auto weights = [&](int v, float (&fw)[EPV]) {
        if constexpr (kKeepW) {
            wv[v].unpack(fw);
        } else {
            WV t;
            t.load(wb, v * LPR + lane, vin[v]);
            t.unpack(fw);
        }
    };
    float acc[VPT][EPV];
#pragma unroll
    for (int v = 0; v < VPT; ++v)
#pragma unroll
        for (int k = 0; k < EPV; ++k) acc[v][k] = 0.f;

    const int64_t step = (int64_t)gridDim.x;
    int64_t row = (int64_t)blockIdx.x;
    // copies of row b into stage s (rows past M: record count 0, read as nothing)
    auto issue = [&](int64_t b, int s) {
        const int64_t bb = b < M ? b : 0;
        const uint32_t bytes = b < M ? row_bytes : 0u;
        const __amdgpu_buffer_rsrc_t xr = Buf(x + bb * N, bytes).r;
        const __amdgpu_buffer_rsrc_t gr = Buf(dy + bb * N, bytes).r;
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            u32x4 *sx = ring + ((s * 2 + 0) * VPT + v) * LPR + wave * 64;
            u32x4 *sg = ring + ((s * 2 + 1) * VPT + v) * LPR + wave * 64;
            // (an array element passed straight to the builtin makes clang drop
            // the kernel's host-side stub without a diagnostic)
            const uint32_t ov = off[v];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void *)sx, 16, ov, 0, 0, RMSN_BWD_LOAD_AUX);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(gr, (lds_void *)sg, 16, ov, 0, 0, RMSN_BWD_LOAD_AUX);
        }
        const __amdgpu_buffer_rsrc_t rr = Buf(rstd + bb, b < M ? 4u : 0u).r;
        // every lane copies (lanes past the first read past the record count)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (lds_void *)(rst + (s * kWaves + wave) * kLdsRstdSlots), 4,
                                                 (uint32_t)(lane & 63) * 4u, 0, 0, 0);
        asm volatile("" ::: "memory");
    };
    // The kept weights are waited for before the prologue (a plain register
    // load; waited for later, the compiler's wait would drain the ring).
    if constexpr (kKeepW) {
#pragma unroll
        for (int v = 0; v < VPT; ++v) wv[v].keep();
    }
    for (int s = 0; s < ST; ++s) issue(row + (int64_t)s * step, s);

    int parity = 0, s = 0, m = 0;
    for (; row < M; row += step) {
        wait_vm<(ST - 1) * L, ST, Q>(m);
        u32x4 xv[VPT], gv[VPT];
        float r;
        {
            const uint32_t ax = lds_off(ring + (s * 2 * VPT) * LPR + lane);
            const uint32_t ag = lds_off(ring + ((s * 2 + 1) * VPT) * LPR + lane);
            // Each statement waits for its own reads: the compiler takes an asm
            // output as ready when the statement ends, and may copy it from
            // then on. (An asm immediate must be a constant expression, and v is
            // a loop index, so the addresses are computed.)
#pragma unroll
            for (int v = 0; v < VPT; ++v) {
                asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                             : "=&v"(xv[v]), "=&v"(gv[v])
                             : "v"(ax + (uint32_t)(v * kVecBytes)), "v"(ag + (uint32_t)(v * kVecBytes))
                             : "memory");
            }
            const uint32_t ar = lds_off(rst + (s * kWaves + wave) * kLdsRstdSlots);
            asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(r) : "v"(ar) : "memory");
        }
        issue(row + (int64_t)ST * step, s);
        s = s + 1 == ST ? 0 : s + 1;
        m = m < ST ? m + 1 : ST;
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            if (!vin[v]) {
                xv[v] = z;
                gv[v] = z;
            }
        }

        float sacc = 0.f;
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            float fx[EPV], fg[EPV], fw[EPV];
            E::unpack(xv[v], fx);
            E::unpack(gv[v], fg);
            weights(v, fw);
#pragma unroll
            for (int k = 0; k < EPV; ++k) {
                sacc = __builtin_fmaf(fg[k] * fw[k], fx[k], sacc);
                acc[v][k] = __builtin_fmaf(fg[k] * fx[k], r, acc[v][k]);
            }
        }
        sacc = row_sum_nf<LPR, LPR>(sacc, slots, parity);
        parity ^= 1;
        const float c = r * (r * (r * (sacc / n)));
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            keep_packed(xv[v]);
            keep_packed(gv[v]);
            if constexpr (kKeepW) wv[v].keep();
        }
        const Buf db(dx + row * N, row_bytes);
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            float fx[EPV], fg[EPV], fw[EPV], o[EPV];
            E::unpack(xv[v], fx);
            E::unpack(gv[v], fg);
            weights(v, fw);
#pragma unroll
            for (int k = 0; k < EPV; ++k) o[k] = __builtin_fmaf(-fx[k], c, r * (fg[k] * fw[k]));
            db.store16<RMSN_BWD_STORE_AUX>(off[v], E::pack(o));
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    const Buf pb(partial + (int64_t)blockIdx.x * ldp, (uint32_t)nvec * (uint32_t)(EPV * 4));
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        if (vin[v]) {
#pragma unroll
            for (int q = 0; q < EPV / 4; ++q) {
                u32x4 o;
                o.x = as_u32(acc[v][4 * q]);
                o.y = as_u32(acc[v][4 * q + 1]);
                o.z = as_u32(acc[v][4 * q + 2]);
                o.w = as_u32(acc[v][4 * q + 3]);
                pb.store16<RMSN_BWD_PARTIAL_AUX>((uint32_t)((v * LPR + lane) * EPV + 4 * q) * 4u, o);
            }
        }
    }
}

}  // namespace rmsn
