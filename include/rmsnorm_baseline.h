/*
 * rmsnorm_baseline.h -- an unfused, multi-kernel RMSNorm, kept beside the
 * fused library as the measured reference point for what fusion saves.
 *
 * hello-gpu "Chapter 13 Fused RMSNorm", section 13.2, and the page
 * "Profiling, GPU utilisation and writing a fused kernel", Problem 15, argue
 * that computing the square, the row sum, the scalar and the scaled output in
 * one kernel avoids re-reading the row from HBM, and that fusing the residual
 * add saves a further round trip; neither page measures the gain. These entry
 * points compute the same values as rmsnorm.h with the work split the way
 * separate library operations would split it. Each kernel on its own is a
 * reasonable one (16-byte coalesced accesses, fp32 arithmetic, no atomics):
 * only the fusion is missing, so the difference in time is the fusion's.
 *
 *   rmsn_unfused_fwd:  kernel 1 reads x and writes rstd (per-row sum of
 *                      squares); kernel 2 reads x again with rstd and w and
 *                      writes y. x crosses the memory bus twice.
 *   rmsn_unfused_bwd:  kernel 1 reads x, dy, w and writes S_i = sum_j
 *                      dy_ij w_j x_ij; kernel 2 reads x, dy, w, rstd, S and
 *                      writes dx; kernel 3 reads x, dy, rstd and writes
 *                      column-block partial sums of dy x rstd; kernel 4 adds
 *                      the partials in a fixed order (rmsnorm_bwd_combine).
 *                      x and dy are read three times. Deterministic.
 *   rmsn_add:          c = a + b rounded once to the activation format (the
 *                      separate residual add: the unfused composition of
 *                      rmsnorm_fwd_residual is rmsn_add then rmsnorm_fwd, and
 *                      of rmsnorm_bwd_residual is rmsnorm_bwd then rmsn_add).
 *
 * Formats, statuses and the row-major [M][N] layout are those of rmsnorm.h.
 * These calls take only the 16-byte vector layout: every pointer 16-byte
 * aligned and N * element size a multiple of 16 (RMSN_EINVAL otherwise).
 * Pointers are device pointers owned by the caller; calls are asynchronous on
 * `stream` (a hipStream_t; NULL for the null stream) and allocate nothing.
 */
#ifndef RMSNORM_BASELINE_H
#define RMSNORM_BASELINE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Unfused forward: rstd (fp32 [M], required) then y [M][N]. */
int rmsn_unfused_fwd(const void *x, const void *w, float eps, int64_t M, int64_t N, int dtype, void *y,
                     float *rstd, void *stream);

/* Workspace of rmsn_unfused_bwd in bytes (S and the dW partials), or a
 * negative status. 0 when M == 0. */
int64_t rmsn_unfused_bwd_workspace_bytes(int64_t M, int64_t N, int dtype);

/* Unfused backward: dx [M][N] and dW (fp32 [N]). workspace: 256-byte
 * aligned, at least rmsn_unfused_bwd_workspace_bytes(M, N, dtype) bytes
 * (RMSN_EWORKSPACE otherwise). With M == 0, dW is set to zero. */
int rmsn_unfused_bwd(const void *x, const void *w, const void *dy, const float *rstd, int64_t M, int64_t N,
                     int dtype, void *dx, float *dw, void *workspace, size_t workspace_bytes, void *stream);

/* c[k] = round(a[k] + b[k]) for k < n, in the activation format of `dtype`.
 * c may alias a or b. */
int rmsn_add(const void *a, const void *b, void *c, int64_t n, int dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* RMSNORM_BASELINE_H */
