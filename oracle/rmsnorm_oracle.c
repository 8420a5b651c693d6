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
 *   sections "The backward pass" and "The naive kernel". The expression
 *   below is written out as the derivative of the forward definition
 *   (d r_i / d x_ik = -r_i^3 x_ik / N); it is also what the page's kernels
 *   compute:
 *       V_ij  = dy_ij * w_j                  (the upstream gradient times the weight)
 *       S_i   = sum_j V_ij * x_ij
 *       dx_ij = r_i * V_ij - x_ij * r_i^3 * S_i / N
 *       dW_j  = sum_i dy_ij * x_ij * r_i     (rows ascending)
 *
 *   Residual-add fusion -- the profiling page, Problem 15 (last paragraph of
 *   the kernel sketch): one kernel that produces both the residual sum and
 *   its normalisation. Read here as the unfused composition it replaces: the
 *   sum is stored in the activation format, h_ij = round(x_ij + res_ij), and
 *   the forward above is applied to h as stored. Its backward receives, next
 *   to dy, the gradient dh flowing into h from the residual branch, and
 *   returns dx_ij = dh_ij + (the dx above, evaluated at h), which is the
 *   gradient of both x and res since h = x + res.
 *
 * The backward recomputes r_i in double from x (or h) and eps; it does not
 * read a device-produced rstd.
 *
 * Storage formats (dtype codes): 0 fp32, 1 bf16 bit patterns, 2 fp64 (used by
 * the finite-difference and library checks), 3 fp16 bit patterns. Weights may
 * have their own format. All widen exactly to double. Outputs are double,
 * except the stored residual sum, which is rounded to the activation format
 * (round to nearest, ties to even) and returned widened to double.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_F64 2
#define ORACLE_F16 3

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static double half_to_double(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int e = (h >> 10) & 0x1f;
    const int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24); /* subnormal: f * 2^-14 * 2^-10 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f | 0x400), e - 25); /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

static double elem(const void *base, int dtype, int64_t idx)
{
    if (dtype == ORACLE_F32)
        return (double)((const float *)base)[idx];
    if (dtype == ORACLE_F64)
        return ((const double *)base)[idx];
    if (dtype == ORACLE_F16)
        return half_to_double(((const uint16_t *)base)[idx]);
    /* bf16 is the top half of an fp32 bit pattern */
    uint32_t u = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * Round v to a binary format with `bits` significant bits, smallest normal
 * exponent emin and largest exponent emax, to nearest with ties to even
 * (nearbyint in the default rounding mode). Below 2^emin the quantum stays
 * 2^(emin - bits + 1) (subnormals). Results of magnitude 2^(emax+1) or more
 * overflow to infinity.
 */
static double round_format(double v, int bits, int emin, int emax)
{
    if (v == 0.0 || !isfinite(v))
        return v;
    int E;
    frexp(v, &E); /* v = m * 2^E, 0.5 <= |m| < 1: leading bit has exponent E-1 */
    int lead = E - 1;
    if (lead < emin)
        lead = emin;
    const int q = lead - (bits - 1);
    const double r = ldexp(nearbyint(ldexp(v, -q)), q);
    if (fabs(r) >= ldexp(1.0, emax + 1))
        return r > 0 ? INFINITY : -INFINITY;
    return r;
}

static double round_storage(double v, int dtype)
{
    switch (dtype) {
    case ORACLE_F32: return round_format(v, 24, -126, 127);
    case ORACLE_BF16: return round_format(v, 8, -126, 127);
    case ORACLE_F16: return round_format(v, 11, -14, 15);
    default: return v; /* fp64 */
    }
}

static int bad_dtype(int d)
{
    return d != ORACLE_F32 && d != ORACLE_BF16 && d != ORACLE_F64 && d != ORACLE_F16;
}

static int bad_args(int dtype, int wdtype, int64_t M, int64_t N, double eps)
{
    if (bad_dtype(dtype) || bad_dtype(wdtype))
        return 1;
    if (M < 0 || N <= 0)
        return 1;
    if (!(eps >= 0.0))
        return 1;
    return 0;
}

/* Element (i, j) of the normalised input: x, or the stored sum round(x + res). */
static double in_elem(const void *x, const void *res, int dtype, int64_t idx)
{
    if (!res)
        return elem(x, dtype, idx);
    return round_storage(elem(x, dtype, idx) + elem(res, dtype, idx), dtype);
}

/* r_i = 1 / sqrt(mean_j v_ij^2 + eps) for one row of the normalised input. */
static double row_r(const void *x, const void *res, int dtype, int64_t i, int64_t N, double eps)
{
    double s = 0.0;
    for (int64_t j = 0; j < N; ++j) {
        double v = in_elem(x, res, dtype, i * N + j);
        s += v * v;
    }
    double ms = s / (double)N;
    return 1.0 / sqrt(ms + eps);
}

/*
 * Forward for the listed rows (all rows 0..M-1 when rows == NULL, and then
 * nrows must equal M). Output row k of y (N doubles) and r[k] belong to input
 * row rows[k]. y may be NULL when only r is wanted. With res != NULL the
 * normalised input is the stored sum round(x + res), written to h (may be
 * NULL). Returns 0, or -1 on bad arguments.
 */
int rmsn_oracle_fwd(const void *x, const void *res, const void *w, int dtype, int wdtype, int64_t M,
                    int64_t N, double eps, const int64_t *rows, int64_t nrows, double *h, double *y,
                    double *r)
{
    if (bad_args(dtype, wdtype, M, N, eps) || !x || !r || (y && !w) || nrows < 0)
        return -1;
    if (!rows && nrows != M)
        return -1;
    for (int64_t k = 0; k < nrows; ++k) {
        int64_t i = rows ? rows[k] : k;
        if (i < 0 || i >= M)
            return -1;
        double ri = row_r(x, res, dtype, i, N, eps);
        r[k] = ri;
        for (int64_t j = 0; j < N; ++j) {
            double v = in_elem(x, res, dtype, i * N + j);
            if (h && res)
                h[k * N + j] = v;
            if (y)
                y[k * N + j] = v * ri * elem(w, wdtype, j);
        }
    }
    return 0;
}

/*
 * Input gradient dx for the listed rows (same row convention as the
 * forward), evaluated at x (or, with res != NULL, at the stored sum
 * round(x + res)); with dh != NULL the gradient dh is added. r (may be NULL)
 * receives the fp64 r_i of each listed row.
 */
int rmsn_oracle_bwd_dx(const void *x, const void *res, const void *w, const void *dy, const void *dh,
                       int dtype, int wdtype, int64_t M, int64_t N, double eps, const int64_t *rows,
                       int64_t nrows, double *dx, double *r)
{
    if (bad_args(dtype, wdtype, M, N, eps) || !x || !w || !dy || !dx || nrows < 0)
        return -1;
    if (!rows && nrows != M)
        return -1;
    for (int64_t k = 0; k < nrows; ++k) {
        int64_t i = rows ? rows[k] : k;
        if (i < 0 || i >= M)
            return -1;
        double ri = row_r(x, res, dtype, i, N, eps);
        if (r)
            r[k] = ri;
        double S = 0.0;
        for (int64_t j = 0; j < N; ++j) {
            double V = elem(dy, dtype, i * N + j) * elem(w, wdtype, j);
            S += V * in_elem(x, res, dtype, i * N + j);
        }
        double ri3 = ri * ri * ri;
        for (int64_t j = 0; j < N; ++j) {
            double V = elem(dy, dtype, i * N + j) * elem(w, wdtype, j);
            double g = ri * V - in_elem(x, res, dtype, i * N + j) * ri3 * S / (double)N;
            dx[k * N + j] = dh ? g + elem(dh, dtype, i * N + j) : g;
        }
    }
    return 0;
}

/* Weight gradient dW_j = sum over all rows i (ascending) of dy_ij * v_ij * r_i,
 * v the normalised input (x, or the stored sum round(x + res)). */
int rmsn_oracle_bwd_dw(const void *x, const void *res, const void *dy, int dtype, int64_t M, int64_t N,
                       double eps, double *dw)
{
    if (bad_args(dtype, dtype, M, N, eps) || !dw || (M > 0 && (!x || !dy)))
        return -1;
    for (int64_t j = 0; j < N; ++j)
        dw[j] = 0.0;
    for (int64_t i = 0; i < M; ++i) {
        double ri = row_r(x, res, dtype, i, N, eps);
        for (int64_t j = 0; j < N; ++j)
            dw[j] += elem(dy, dtype, i * N + j) * in_elem(x, res, dtype, i * N + j) * ri;
    }
    return 0;
}

/* The storage rounding on its own, for its pins: out[k] = round(in[k]) in `dtype`. */
int rmsn_oracle_round(const double *in, int64_t n, int dtype, double *out)
{
    if (bad_dtype(dtype) || n < 0 || (n > 0 && (!in || !out)))
        return -1;
    for (int64_t k = 0; k < n; ++k)
        out[k] = round_storage(in[k], dtype);
    return 0;
}
