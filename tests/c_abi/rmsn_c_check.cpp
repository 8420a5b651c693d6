// rmsn_c_check.cpp -- TEST PROGRAM: the library driven through its C ABI
// alone (include/rmsnorm.h), with no Python and no torch in the process, and
// its results checked against the fp64 CPU oracle (oracle/rmsnorm_oracle.c,
// linked in; test code may use it, the library never does).
//
// For a few shapes (bf16 and fp32, aligned and ragged), it generates seeded
// inputs, runs rmsnorm_fwd and rmsnorm_bwd on plain hipMalloc buffers, and
// checks every element of y, rstd, dx and dW against the oracle. The gates
// match the Python parity tests:
//   y, dx fp32: |g-o| <= 1e-5 * max(|o|, row rms of o, row rms of r*dy*w)
//   y, dx bf16: |g-o| <= 2^-7 * (|o| + 0.01 * that row rms)
//   rstd:       |g-o| <= 1e-5 * o;   dW: |g-o| <= tol * max(|o|, floor * rms(dW))
// Prints "ok" and exits 0 when every check passes, nonzero otherwise.
// With --host-timing it instead reports the host time per call of the entry
// points at decode-sized shapes (M = 1, 2, 4 rows of 4096 bf16 columns).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "../../include/rmsnorm.h"

extern "C" {
int rmsn_oracle_fwd(const void *x, const void *res, const void *w, int dtype, int wdtype, int64_t M, int64_t N,
                    double eps, const int64_t *rows, int64_t nrows, double *h, double *y, double *r);
int rmsn_oracle_bwd_dx(const void *x, const void *res, const void *w, const void *dy, const void *dh, int dtype,
                       int wdtype, int64_t M, int64_t N, double eps, const int64_t *rows, int64_t nrows, double *dx,
                       double *r);
int rmsn_oracle_bwd_dw(const void *x, const void *res, const void *dy, int dtype, int64_t M, int64_t N, double eps,
                       double *dw);
}

namespace {

constexpr int kOracleF32 = 0, kOracleBf16 = 1;

// SplitMix64 (Steele, Lea, Flood 2014) -> uniform doubles -> normals by Box-Muller:
// seeded inputs only, no arithmetic of the method.
struct Rng {
    uint64_t s;
    uint64_t next() {
        uint64_t z = (s += 0x9E3779B97F4A7C15ull);
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        return z ^ (z >> 31);
    }
    double uniform() { return ((next() >> 11) + 0.5) * (1.0 / 9007199254740992.0); }
    double normal() { return std::sqrt(-2.0 * std::log(uniform())) * std::cos(6.283185307179586 * uniform()); }
};

uint16_t to_bf16(float f) {  // round to nearest even on the bit pattern (finite inputs)
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
double from_bf16(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

#define HIP_OK(call)                                                                   \
    do {                                                                               \
        hipError_t e_ = (call);                                                        \
        if (e_ != hipSuccess) {                                                        \
            std::fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));   \
            return false;                                                              \
        }                                                                              \
    } while (0)

int g_failures = 0;

void gate_rows(const char *what, const std::vector<double> &g, const std::vector<double> &o,
               const std::vector<double> &floor_rms, int64_t M, int64_t N, bool bf16) {
    for (int64_t i = 0; i < M; ++i) {
        double ss = 0;
        for (int64_t j = 0; j < N; ++j) ss += o[i * N + j] * o[i * N + j];
        double rms = std::sqrt(ss / (double)N);
        if (!floor_rms.empty() && floor_rms[i] > rms) rms = floor_rms[i];
        for (int64_t j = 0; j < N; ++j) {
            const double ov = o[i * N + j], gv = g[i * N + j], err = std::fabs(gv - ov);
            const double bound = bf16 ? std::ldexp(1.0, -7) * (std::fabs(ov) + 0.01 * rms)
                                      : 1e-5 * std::fmax(std::fabs(ov), rms);
            if (!(err <= bound)) {
                if (g_failures++ < 10)
                    std::printf("FAIL %s[%lld][%lld]: gpu %.9g oracle %.9g bound %.3g\n", what, (long long)i,
                                (long long)j, gv, ov, bound);
            }
        }
    }
}

template <typename S>
bool run_case(int64_t M, int64_t N, bool bf16, uint64_t seed) {
    const int dtype = bf16 ? RMSN_BF16 : RMSN_F32;
    const int odt = bf16 ? kOracleBf16 : kOracleF32;
    const float eps = 1e-6f;
    Rng rng{seed};
    std::vector<S> x(M * N), dy(M * N), w(N);
    auto store = [&](double v) -> S {
        if constexpr (sizeof(S) == 2) return (S)to_bf16((float)v);
        else return (S)(float)v;
    };
    auto load = [&](S v) -> double {
        if constexpr (sizeof(S) == 2) return from_bf16((uint16_t)v);
        else return (double)v;
    };
    for (auto &v : x) v = store(rng.normal());
    for (auto &v : w) v = store(1.0 + 0.1 * rng.normal());
    for (auto &v : dy) v = store((bf16 ? 1e-2 : 1.0) * rng.normal());

    const size_t bytes = (size_t)M * N * sizeof(S);
    S *dx_d, *dy_d, *y_d, *dxo_d, *w_d;
    float *rstd_d, *dw_d;
    void *ws_d = nullptr;
    HIP_OK(hipMalloc(&dx_d, bytes));
    HIP_OK(hipMalloc(&dy_d, bytes));
    HIP_OK(hipMalloc(&y_d, bytes));
    HIP_OK(hipMalloc(&dxo_d, bytes));
    HIP_OK(hipMalloc(&w_d, N * sizeof(S)));
    HIP_OK(hipMalloc(&rstd_d, M * sizeof(float)));
    HIP_OK(hipMalloc(&dw_d, N * sizeof(float)));
    HIP_OK(hipMemcpy(dx_d, x.data(), bytes, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dy_d, dy.data(), bytes, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(w_d, w.data(), N * sizeof(S), hipMemcpyHostToDevice));

    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    int st = rmsnorm_fwd(dx_d, w_d, eps, M, N, dtype, y_d, rstd_d, stream);
    if (st != RMSN_OK) {
        std::printf("FAIL rmsnorm_fwd: %s\n", rmsnorm_status_str(st));
        return false;
    }
    const int64_t need = rmsnorm_bwd_workspace_bytes(M, N, dtype);
    if (need < 0) {
        std::printf("FAIL workspace query: %s\n", rmsnorm_status_str((int)need));
        return false;
    }
    HIP_OK(hipMalloc(&ws_d, need > 0 ? (size_t)need : 256));
    st = rmsnorm_bwd(dx_d, w_d, dy_d, rstd_d, M, N, dtype, dxo_d, dw_d, ws_d, (size_t)need, stream);
    if (st != RMSN_OK) {
        std::printf("FAIL rmsnorm_bwd: %s\n", rmsnorm_status_str(st));
        return false;
    }
    HIP_OK(hipStreamSynchronize(stream));

    std::vector<S> y(M * N), dxg(M * N);
    std::vector<float> rstd(M), dw(N);
    HIP_OK(hipMemcpy(y.data(), y_d, bytes, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(dxg.data(), dxo_d, bytes, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(rstd.data(), rstd_d, M * sizeof(float), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(dw.data(), dw_d, N * sizeof(float), hipMemcpyDeviceToHost));

    std::vector<double> oy(M * N), odx(M * N), orr(M), odw(N);
    if (rmsn_oracle_fwd(x.data(), nullptr, w.data(), odt, odt, M, N, eps, nullptr, M, nullptr, oy.data(),
                        orr.data()) != 0 ||
        rmsn_oracle_bwd_dx(x.data(), nullptr, w.data(), dy.data(), nullptr, odt, odt, M, N, eps, nullptr, M,
                           odx.data(), nullptr) != 0 ||
        rmsn_oracle_bwd_dw(x.data(), nullptr, dy.data(), odt, M, N, eps, odw.data()) != 0) {
        std::printf("FAIL oracle rejected its arguments\n");
        return false;
    }
    const int before = g_failures;
    std::vector<double> gy(M * N), gdx(M * N), trms(M);
    for (int64_t k = 0; k < M * N; ++k) {
        gy[k] = load(y[k]);
        gdx[k] = load(dxg[k]);
    }
    for (int64_t i = 0; i < M; ++i) {  // rms of r * dy * w per row: the size of the terms dx cancels
        double ss = 0;
        for (int64_t j = 0; j < N; ++j) {
            const double t = orr[i] * load(dy[i * N + j]) * load(w[j]);
            ss += t * t;
        }
        trms[i] = std::sqrt(ss / (double)N);
    }
    gate_rows("y", gy, oy, {}, M, N, bf16);
    gate_rows("dx", gdx, odx, trms, M, N, bf16);
    for (int64_t i = 0; i < M; ++i)
        if (!(std::fabs(rstd[i] - orr[i]) <= 1e-5 * orr[i]) && g_failures++ < 10)
            std::printf("FAIL rstd[%lld]: gpu %.9g oracle %.9g\n", (long long)i, rstd[i], orr[i]);
    double ss = 0;
    for (int64_t j = 0; j < N; ++j) ss += odw[j] * odw[j];
    const double rms = std::sqrt(ss / (double)N);
    for (int64_t j = 0; j < N; ++j) {
        const double bound = bf16 ? 1e-3 * std::fmax(std::fabs(odw[j]), 1e-2 * rms)
                                  : 1e-5 * std::fmax(std::fabs(odw[j]), rms);
        if (!(std::fabs(dw[j] - odw[j]) <= bound) && g_failures++ < 10)
            std::printf("FAIL dW[%lld]: gpu %.9g oracle %.9g\n", (long long)j, dw[j], odw[j]);
    }
    std::printf("%s %lldx%lld: %s\n", bf16 ? "bf16" : "fp32", (long long)M, (long long)N,
                g_failures == before ? "pass" : "FAIL");
    for (void *p : {(void *)dx_d, (void *)dy_d, (void *)y_d, (void *)dxo_d, (void *)w_d, (void *)rstd_d,
                    (void *)dw_d, ws_d})
        (void)hipFree(p);
    (void)hipStreamDestroy(stream);
    return g_failures == before;
}

// Host time per call (no Python in the process): batches of kBatch calls are
// issued back to back and timed on the host clock around the issuing only;
// the stream is drained between batches (untimed) so the launch queue never
// fills and blocks the caller. Reported: the median over batches of the time
// per call, for rmsnorm_bwd (argument checks, the cached configuration and
// workspace lookups, one or two launches), rmsnorm_fwd, and, for scale,
// rmsnorm_bwd_combine (argument checks and a single launch, no lookup).
bool host_timing() {
    constexpr int kBatch = 200, kBatches = 25;
    const int64_t N = 4096;
    uint16_t *x, *dy, *dx, *w, *y;
    float *rstd, *dw;
    void *ws;
    const size_t elems = 4 * N;
    HIP_OK(hipMalloc(&x, elems * 2));
    HIP_OK(hipMalloc(&dy, elems * 2));
    HIP_OK(hipMalloc(&dx, elems * 2));
    HIP_OK(hipMalloc(&y, elems * 2));
    HIP_OK(hipMalloc(&w, N * 2));
    HIP_OK(hipMalloc(&rstd, 4 * sizeof(float)));
    HIP_OK(hipMalloc(&dw, N * sizeof(float)));
    HIP_OK(hipMemset(x, 0x3f, elems * 2));
    HIP_OK(hipMemset(dy, 0x3c, elems * 2));
    HIP_OK(hipMemset(w, 0x3f, N * 2));
    const size_t ws_bytes = 64u << 20;
    HIP_OK(hipMalloc(&ws, ws_bytes));
    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));
    auto time_calls = [&](const char *what, int64_t M, auto &&call) -> bool {
        std::vector<double> per;
        for (int b = 0; b < kBatches + 2; ++b) {
            const auto t0 = std::chrono::steady_clock::now();
            for (int i = 0; i < kBatch; ++i)
                if (call(M) != RMSN_OK) {
                    std::printf("FAIL %s returned an error\n", what);
                    return false;
                }
            const auto t1 = std::chrono::steady_clock::now();
            if (hipStreamSynchronize(s) != hipSuccess) return false;
            if (b >= 2) per.push_back(std::chrono::duration<double, std::micro>(t1 - t0).count() / kBatch);
        }
        std::sort(per.begin(), per.end());
        std::printf("host time per call: %s M=%lld N=%lld bf16: median %.2f us (min %.2f, max %.2f) over %d x %d calls\n",
                    what, (long long)M, (long long)N, per[per.size() / 2], per.front(), per.back(), kBatches, kBatch);
        return true;
    };
    bool ok = true;
    for (int64_t M : {1, 2, 4}) {
        ok &= time_calls("rmsnorm_bwd", M, [&](int64_t m) {
            return rmsnorm_bwd(x, w, dy, rstd, m, N, RMSN_BF16, dx, dw, ws, ws_bytes, s);
        });
        ok &= time_calls("rmsnorm_fwd", M, [&](int64_t m) {
            return rmsnorm_fwd(x, w, 1e-6f, m, N, RMSN_BF16, y, rstd, s);
        });
    }
    ok &= time_calls("rmsnorm_bwd_combine", 1, [&](int64_t) { return rmsnorm_bwd_combine(ws, 1, N, dw, s); });
    for (void *p : {(void *)x, (void *)dy, (void *)dx, (void *)y, (void *)w, (void *)rstd, (void *)dw, ws}) (void)hipFree(p);
    (void)hipStreamDestroy(s);
    return ok;
}

}  // namespace

int main(int argc, char **argv) {
    if (argc > 1 && std::strcmp(argv[1], "--host-timing") == 0) {
        int dev = 0;
        if (hipGetDeviceCount(&dev) != hipSuccess || dev < 1) {
            std::printf("FAIL no HIP device\n");
            return 2;
        }
        const bool ok = host_timing();
        std::printf("%s\n", ok ? "ok" : "FAILED");
        return ok ? 0 : 1;
    }
    int dev = 0;
    if (hipGetDeviceCount(&dev) != hipSuccess || dev < 1) {
        std::printf("FAIL no HIP device\n");
        return 2;
    }
    std::printf("%s\n", rmsnorm_build_info());
    bool ok = true;
    ok &= run_case<uint16_t>(257, 4096, true, 1);    // vector path, ragged row count
    ok &= run_case<uint16_t>(64, 32768, true, 2);    // wide-row backward
    ok &= run_case<uint16_t>(40, 65536, true, 9);    // split-row backward (exchange slots in the workspace)
    ok &= run_case<float>(6, 131072, false, 10);     // two-pass forward, split fp32 backward
    ok &= run_case<uint16_t>(1000, 128, true, 3);    // several rows per wavefront
    ok &= run_case<float>(33, 257, false, 4);        // element kernels (row not a multiple of 16 bytes)
    ok &= run_case<uint16_t>(9, 4100, true, 6);      // element kernels, 4 elements per access
    ok &= run_case<float>(7, 13, false, 7);          // element kernels, 64-lane rows
    ok &= run_case<float>(3, 16385, false, 8);       // scalar path (wider than the element kernels hold)
    ok &= run_case<float>(96, 1024, false, 5);
    std::printf("%s\n", ok ? "ok" : "FAILED");
    return ok ? 0 : 1;
}
