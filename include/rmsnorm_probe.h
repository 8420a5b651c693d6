/*
 * rmsnorm_probe.h -- HBM roofline probes used by the benchmark.
 *
 * The achievable-bandwidth denominator is measured, not quoted: the best of
 * a copy, a pure write and a two-read-one-write pattern ("What a tuned
 * RMSNorm kernel actually costs on Hopper", section 02). Each probe streams
 * 16-byte vectors over caller-owned device buffers; `bytes` must be a
 * multiple of 16 and every pointer 16-byte aligned. `grid` is the number of
 * 256-lane workgroups (0 = one vector per lane, no striding). `variant`
 * selects the cache hint: bit 0 non-temporal loads, bit 1 non-temporal
 * stores (0..3). Work is enqueued on `stream` (a hipStream_t; NULL = default
 * stream). Returns 0 or a negative rmsn_status (see rmsnorm.h).
 */
#ifndef RMSNORM_MI355X_PROBE_H
#define RMSNORM_MI355X_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dst[i] = src[i]: moves 2 * bytes (one read, one write). */
int rmsn_probe_copy(const void *src, void *dst, size_t bytes, int64_t grid, int variant, void *stream);

/* dst[i] = pattern: moves `bytes` (write only). */
int rmsn_probe_write(void *dst, size_t bytes, int64_t grid, int variant, void *stream);

/* Reads src (moves `bytes`); writes at most 16 bytes to sink (device memory,
 * 16-byte aligned). Used as a cache flush that leaves no dirty lines behind. */
int rmsn_probe_read(const void *src, size_t bytes, int64_t grid, int variant, void *sink, void *stream);

/* c[i] = a[i] + b[i] as 32-bit integers: moves 3 * bytes (two reads, one write). */
int rmsn_probe_add(const void *a, const void *b, void *c, size_t bytes, int64_t grid, int variant,
                   void *stream);

#ifdef __cplusplus
}
#endif

#endif /* RMSNORM_MI355X_PROBE_H */
