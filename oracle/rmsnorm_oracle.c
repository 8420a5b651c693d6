/*
 * rmsnorm_oracle.c -- plain, slow, fp64 CPU oracle for RMSNorm forward and
 * backward.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this code. The GPU library neither links
 * nor calls it, and shares no source with it.
 *
 * What it computes (every sum in double, index ascending, no blocking, no
 * reordering):
 *
 *   Forward -- hello-gpu "Chapter 13 Fused RMSNorm", section 13.1 (the
 *   definition and the worked examples); the same definition appears in the
 *   page "Profiling, GPU utilisation and writing a fused kernel", Problem 15
 *   ("The concepts"):
 *       ms_i = (1/N) * sum_j x_ij^2          (N = true column count)
 *       r_i  = 1 / sqrt(ms_i + eps)          (eps inside the root)
 *       y_ij = x_ij * r_i * w_j              (w is per column, shared by rows)
 *
 *   Backward -- "RMSNorm backward (almost) without the column reduction",
 *   sections "The backward pass" and "The naive kernel". The page's formula
 *   images are lost; the expression below is the derivative of the forward
 *   definition (d r_i / d x_ik = -r_i^3 x_ik / N), which is also what the
 *   page's kernels compute:
 *       V_ij  = dy_ij * w_j                  ("incoming gradient after the gain")
 *       S_i   = sum_j V_ij * x_ij
 *       dx_ij = r_i * V_ij - x_ij * r_i^3 * S_i / N
 *       dW_j  = sum_i dy_ij * x_ij * r_i     (rows ascending)
 *
 * The backward recomputes r_i in double from x and eps (it does not read a
 * device-produced rstd).
 *
 * Inputs are in storage format: dtype 0 = fp32, dtype 1 = bf16 bit patterns
 * (uint16), dtype 2 = fp64 (used by the finite-difference and library checks).
 * All widen exactly to double. Outputs are double.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_F64 2

static double elem(const void *base, int dtype, int64_t idx)
{
    if (dtype == ORACLE_F32)
        return (double)((const float *)base)[idx];
    if (dtype == ORACLE_F64)
        return ((const double *)base)[idx];
    /* bf16 is the top half of an fp32 bit pattern */
    uint32_t u = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static int bad_args(int dtype, int64_t M, int64_t N, double eps)
{
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16 && dtype != ORACLE_F64)
        return 1;
    if (M < 0 || N <= 0)
        return 1;
    if (!(eps >= 0.0))
        return 1;
    return 0;
}

/* r_i = 1 / sqrt(mean_j x_ij^2 + eps) for one row. */
static double row_r(const void *x, int dtype, int64_t i, int64_t N, double eps)
{
    double s = 0.0;
    for (int64_t j = 0; j < N; ++j) {
        double v = elem(x, dtype, i * N + j);
        s += v * v;
    }
    double ms = s / (double)N;
    return 1.0 / sqrt(ms + eps);
}

/*
 * Forward for the listed rows (all rows 0..M-1 when rows == NULL, and then
 * nrows must equal M). Output row k of y (N doubles) and r[k] belong to input
 * row rows[k]. y may be NULL when only r is wanted. Returns 0, or -1 on bad
 * arguments.
 */
int rmsn_oracle_fwd(const void *x, const void *w, int dtype, int64_t M, int64_t N,
                    double eps, const int64_t *rows, int64_t nrows, double *y,
                    double *r)
{
    if (bad_args(dtype, M, N, eps) || !x || !r || (y && !w) || nrows < 0)
        return -1;
    if (!rows && nrows != M)
        return -1;
    for (int64_t k = 0; k < nrows; ++k) {
        int64_t i = rows ? rows[k] : k;
        if (i < 0 || i >= M)
            return -1;
        double ri = row_r(x, dtype, i, N, eps);
        r[k] = ri;
        if (y) {
            for (int64_t j = 0; j < N; ++j)
                y[k * N + j] = elem(x, dtype, i * N + j) * ri * elem(w, dtype, j);
        }
    }
    return 0;
}

/*
 * Input gradient dx for the listed rows (same row convention as the forward).
 * r (may be NULL) receives the fp64 r_i of each listed row.
 */
int rmsn_oracle_bwd_dx(const void *x, const void *w, const void *dy, int dtype,
                       int64_t M, int64_t N, double eps, const int64_t *rows,
                       int64_t nrows, double *dx, double *r)
{
    if (bad_args(dtype, M, N, eps) || !x || !w || !dy || !dx || nrows < 0)
        return -1;
    if (!rows && nrows != M)
        return -1;
    for (int64_t k = 0; k < nrows; ++k) {
        int64_t i = rows ? rows[k] : k;
        if (i < 0 || i >= M)
            return -1;
        double ri = row_r(x, dtype, i, N, eps);
        if (r)
            r[k] = ri;
        double S = 0.0;
        for (int64_t j = 0; j < N; ++j) {
            double V = elem(dy, dtype, i * N + j) * elem(w, dtype, j);
            S += V * elem(x, dtype, i * N + j);
        }
        double ri3 = ri * ri * ri;
        for (int64_t j = 0; j < N; ++j) {
            double V = elem(dy, dtype, i * N + j) * elem(w, dtype, j);
            dx[k * N + j] = ri * V - elem(x, dtype, i * N + j) * ri3 * S / (double)N;
        }
    }
    return 0;
}

/* Weight gradient dW_j = sum over all rows i (ascending) of dy_ij * x_ij * r_i. */
int rmsn_oracle_bwd_dw(const void *x, const void *dy, int dtype, int64_t M, int64_t N,
                       double eps, double *dw)
{
    if (bad_args(dtype, M, N, eps) || !dw || (M > 0 && (!x || !dy)))
        return -1;
    for (int64_t j = 0; j < N; ++j)
        dw[j] = 0.0;
    for (int64_t i = 0; i < M; ++i) {
        double ri = row_r(x, dtype, i, N, eps);
        for (int64_t j = 0; j < N; ++j)
            dw[j] += elem(dy, dtype, i * N + j) * elem(x, dtype, i * N + j) * ri;
    }
    return 0;
}
