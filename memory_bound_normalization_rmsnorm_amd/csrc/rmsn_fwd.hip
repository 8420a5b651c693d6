// rmsn_fwd.hip -- RMSNorm forward kernels for gfx950.
//
// Per row i: rstd_i = 1/sqrt(sum_j x_ij^2 / N + eps), y_ij = x_ij * rstd_i * w_j
// (hello-gpu "Chapter 13 Fused RMSNorm", section 13.1). The square, the row
// sum, the scalar and the scaled store happen in one kernel with the row
// held in registers, so x is read from HBM exactly once (the chapter's
// section 13.2 notes that fusing alone does not guarantee a single read).
//
// Vector kernel: a row is shared by LPR lanes; lane l holds the 16-byte
// vectors l, l + LPR, l + 2*LPR, ... (VPT of them), so each load instruction
// of a row group covers LPR * 16 contiguous bytes. Accesses go through a
// buffer resource per row block whose record count covers only the rows that
// exist; vectors past the row end use an out-of-range offset. Such lanes load
// zeros (adding nothing to the sum) and store nothing; the mean always
// divides by the true N. A workgroup of WG = max(LPR, 256) lanes works on
// WG / LPR rows at a time and strides over rows by grid * (WG / LPR); w is
// loaded into registers once per workgroup.
//
// Scalar kernel: any N and any alignment; one workgroup of 256 lanes per row,
// strided fp32/bf16 element loads, x re-read (from cache) for the output.
#include "rmsn_device.h"
#include "rmsn_tables.h"

namespace rmsn {

template <typename T, int LPR, int VPT, int WG>
__global__ void __launch_bounds__(WG)
__attribute__((amdgpu_waves_per_eu(waves_for(2 * VPT, 0, VPT, WG))))
fwd_vec(const T *__restrict__ x, const T *__restrict__ w, T *__restrict__ y,
        float *__restrict__ rstd, float eps, int64_t M, int32_t N, int32_t nvec) {
    using E = Elem<T>;
    constexpr int RPW = WG / LPR;
    static_assert(WG % LPR == 0, "workgroup must hold whole row groups");
    __shared__ float slots[LPR > 64 ? 2 * (WG / 64) : 1];

    const int lane = threadIdx.x % LPR;
    const int grp = threadIdx.x / LPR;
    const float n = (float)N;
    const uint32_t row_bytes = (uint32_t)nvec * 16u;

    // Byte offset of each of this lane's vectors inside a row block; vectors
    // past the row end get an out-of-range offset.
    uint32_t off[VPT];
    const Buf wb(w, row_bytes);
    u32x4 wv[VPT];
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
        const int idx = v * LPR + lane;
        const bool in = idx < nvec;
        off[v] = in ? (uint32_t)grp * row_bytes + (uint32_t)idx * 16u : kOff;
        wv[v] = wb.load16(in ? (uint32_t)idx * 16u : kOff);
    }

    int parity = 0;
    const int64_t step = (int64_t)gridDim.x * RPW;
    for (int64_t base = (int64_t)blockIdx.x * RPW; base < M; base += step) {
        const int64_t left = M - base;
        const uint32_t rows = left < RPW ? (uint32_t)left : (uint32_t)RPW;
        const Buf xb(x + base * N, rows * row_bytes);
        const Buf yb(y + base * N, rows * row_bytes);
#pragma unroll
        for (int v = 0; v < VPT; ++v) keep_packed(wv[v]);

        u32x4 xv[VPT];
#pragma unroll
        for (int v = 0; v < VPT; ++v) xv[v] = xb.load16(off[v]);

        float ss = 0.f;
#pragma unroll
        for (int v = 0; v < VPT; ++v) ss = E::sumsq(xv[v], ss);
        ss = row_sum<LPR, WG>(ss, slots, parity);
        parity ^= 1;
        const float r = __frsqrt_rn(ss / n + eps);

        if (rstd) {
            const Buf rb(rstd + base, rows * 4u);
            rb.store4(lane == 0 ? (uint32_t)grp * 4u : kOff, r);
        }
#pragma unroll
        for (int v = 0; v < VPT; ++v) keep_packed(xv[v]);
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
            float f[E::kPerVec], g[E::kPerVec];
            E::unpack(xv[v], f);
            E::unpack(wv[v], g);
#pragma unroll
            for (int k = 0; k < E::kPerVec; ++k) f[k] = (f[k] * r) * g[k];
            yb.store16(off[v], E::pack(f));
        }
    }
}

template <typename T>
__global__ void __launch_bounds__(kScalarWG)
fwd_scalar(const T *__restrict__ x, const T *__restrict__ w, T *__restrict__ y,
           float *__restrict__ rstd, float eps, int64_t M, int32_t N, int32_t /*nvec*/) {
    using E = Elem<T>;
    __shared__ float slots[2 * (kScalarWG / 64)];
    const float n = (float)N;
    int parity = 0;
    for (int64_t row = blockIdx.x; row < M; row += gridDim.x) {
        const T *xr = x + row * (int64_t)N;
        float ss = 0.f;
        for (int j = threadIdx.x; j < N; j += kScalarWG) {
            const float f = E::load(xr + j);
            ss = __builtin_fmaf(f, f, ss);
        }
        ss = row_sum<kScalarWG, kScalarWG>(ss, slots, parity);
        parity ^= 1;
        const float r = __frsqrt_rn(ss / n + eps);
        if (threadIdx.x == 0 && rstd) rstd[row] = r;
        T *yr = y + row * (int64_t)N;
        for (int j = threadIdx.x; j < N; j += kScalarWG) E::store(yr + j, (E::load(xr + j) * r) * E::load(w + j));
    }
}

// ---- dispatch tables -------------------------------------------------------

#define RMSN_FWD(T, L, V) {L, V, wg_for_lpr(L), reinterpret_cast<const void *>(&fwd_vec<T, L, V, wg_for_lpr(L)>)}
#define RMSN_FWD_VPT(T, L)                                                                      \
    RMSN_FWD(T, L, 1), RMSN_FWD(T, L, 2), RMSN_FWD(T, L, 3), RMSN_FWD(T, L, 4), RMSN_FWD(T, L, 5), \
        RMSN_FWD(T, L, 6), RMSN_FWD(T, L, 7), RMSN_FWD(T, L, 8)
#define RMSN_FWD_ALL(T)                                                                           \
    RMSN_FWD(T, 1, 1), RMSN_FWD(T, 2, 1), RMSN_FWD(T, 4, 1), RMSN_FWD(T, 8, 1), RMSN_FWD(T, 16, 1), \
        RMSN_FWD(T, 32, 1), RMSN_FWD_VPT(T, 64), RMSN_FWD_VPT(T, 128), RMSN_FWD_VPT(T, 256),      \
        RMSN_FWD_VPT(T, 512), RMSN_FWD_VPT(T, 1024)

static const KernelEntry kFwdF32[] = {RMSN_FWD_ALL(float)};
static const KernelEntry kFwdBf16[] = {RMSN_FWD_ALL(bf16_t)};

const KernelEntry *fwd_vec_kernel(int dtype, int lpr, int vpt) {
    const KernelEntry *t = dtype == 0 ? kFwdF32 : kFwdBf16;
    const int n = dtype == 0 ? (int)(sizeof(kFwdF32) / sizeof(kFwdF32[0]))
                             : (int)(sizeof(kFwdBf16) / sizeof(kFwdBf16[0]));
    for (int i = 0; i < n; ++i)
        if (t[i].lpr == lpr && t[i].vpt == vpt) return &t[i];
    return nullptr;
}

const void *fwd_scalar_kernel(int dtype) {
    return dtype == 0 ? reinterpret_cast<const void *>(&fwd_scalar<float>)
                      : reinterpret_cast<const void *>(&fwd_scalar<bf16_t>);
}

}  // namespace rmsn
