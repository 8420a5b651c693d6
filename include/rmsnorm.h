/*
 * rmsnorm.h -- C ABI of the MI355X (gfx950) RMSNorm library.
 *
 * Forward: for each row i of an M x N row-major matrix x,
 *     rstd_i = 1 / sqrt((1/N) * sum_j x_ij^2 + eps)      (eps inside the root,
 *     y_ij   = x_ij * rstd_i * w_j                          N the true width)
 * as defined in hello-gpu "Chapter 13 Fused RMSNorm", section 13.1, and in the
 * page "Profiling, GPU utilisation and writing a fused kernel", Problem 15
 * ("The concepts").
 *
 * Backward: with V_ij = dy_ij * w_j, the upstream gradient scaled by the
 * weight ("RMSNorm backward (almost) without the column reduction", section
 * "The backward pass"),
 *     dx_ij = rstd_i * V_ij - x_ij * rstd_i^3 * (sum_j V_ij x_ij) / N
 *     dW_j  = sum_i dy_ij * x_ij * rstd_i
 * This is the derivative of the forward, written out here; it matches what
 * the page's kernels compute. dW is reduced without atomics in a fixed
 * order, so it is bit-identical from run to run on the same device (same
 * page, section "The problem: summing across rows"). The backward reads the
 * fp32 rstd the forward wrote, as the Quack study describes its backward
 * ("What a tuned RMSNorm kernel actually costs on Hopper", section 05).
 *
 * Conventions for every entry point:
 *   - `dtype` is an rmsn_dtype: the activation format of x, y, dy, dx (and
 *     res, h, dh) and the weight format of w; rstd, dW and the workspace are
 *     always fp32.
 *   - All tensor pointers are DEVICE pointers, allocated and owned by the
 *     caller. Matrices are row-major and contiguous (row stride = N
 *     elements); w and dW have N elements; rstd has M elements.
 *   - The library allocates nothing. Its only state is a per-device cache of
 *     properties (compute-unit count, kernel occupancy).
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *     default stream). Nothing synchronises the host.
 *   - Argument checks run before any HIP call. M == 0 is a valid no-op.
 *   - Any N >= 1 is accepted. Every pointer must be aligned to its element
 *     type (2 or 4 bytes; rstd and dW 4; RMSN_EINVAL otherwise). 16-byte vector loads are
 *     used when N * sizeof(elem) is a multiple of 16 and every matrix/vector
 *     pointer is 16-byte aligned; otherwise kernels of the same arithmetic
 *     with narrower accesses run (rows of up to 16384 columns: groups of
 *     consecutive elements as wide as N and the pointers' alignment allow;
 *     wider rows: one element per access).
 *   - y must not alias x; dx must not alias x or dy (undefined behaviour).
 *   - Return value: RMSN_OK (0) or a negative rmsn_status.
 */
#ifndef RMSNORM_MI355X_H
#define RMSNORM_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Storage formats: activations (x, y, dy, dx, and the residual tensors) and
 * weights w. 16-bit outputs are rounded to nearest even. rstd, dW and the
 * workspace are fp32 in every format. The *_WF32 formats keep fp32 (master)
 * weights with 16-bit activations ("What a tuned RMSNorm kernel actually costs
 * on Hopper", section 07: weight format as a separate dimension).
 */
typedef enum {
    RMSN_F32 = 0,       /* fp32 activations, fp32 weights */
    RMSN_BF16 = 1,      /* bf16 activations, bf16 weights */
    RMSN_F16 = 2,       /* fp16 activations, fp16 weights */
    RMSN_BF16_WF32 = 3, /* bf16 activations, fp32 weights */
    RMSN_F16_WF32 = 4   /* fp16 activations, fp32 weights */
} rmsn_dtype;

typedef enum {
    RMSN_OK = 0,
    RMSN_EINVAL = -1,      /* null pointer, M < 0, N < 1, eps < 0 or not finite, size overflow */
    RMSN_EDTYPE = -2,      /* dtype is not an rmsn_dtype */
    RMSN_EWORKSPACE = -3,  /* workspace null or smaller than rmsnorm_bwd_workspace_bytes() */
    RMSN_EHIP = -4,        /* a HIP runtime call or kernel launch failed */
    RMSN_ECONFIG = -5,     /* an explicit launch configuration does not fit the shape */
    RMSN_ESCRATCH = -6     /* rmsnorm_bwd_noalloc: the shape needs more than the static workspace */
} rmsn_status;

/*
 * Launch configuration chosen by the library's ladder (keyed on the row
 * width, as the Quack analytical ladder is: "What a tuned RMSNorm kernel
 * actually costs on Hopper", section 03). Reported for logs and tests.
 */
typedef struct {
    int32_t vector_path;     /* 1: 16-byte vector row kernel; 2: the backward's wide-row vector
                                kernel (1024 lanes, dW sums in LDS); 4: the backward's split-row
                                kernel (each row on K = lanes_per_row / 1024 workgroups of 1024
                                lanes, K = 2..16, that exchange their parts of the row sum
                                through the workspace; vecs_per_lane vectors per lane of each
                                member's slice, 3-4 for 16-bit and 5-8 for fp32 activations;
                                grid a multiple of K, at most what stays resident on the
                                device at once); 5: the forward's two-pass kernel (rows
                                wider than 16 vectors per lane on 1024 lanes, 8 with the
                                residual add: one row per 1024-lane workgroup, read in chunks
                                of vecs_per_lane vectors per lane; the first kept_vecs vectors
                                per lane stay in registers between the passes, with copy_mode 1
                                the next 8 in LDS, and the rest is read twice); 3: element
                                kernel (rows
                                that are not a multiple of 16 bytes or not 16-byte aligned,
                                up to 16384 columns: lanes_per_row = wg_threads = 64, 128, 256,
                                512 or 1024, vecs_per_lane accesses of elems_per_access
                                elements per lane); 0: scalar row kernel */
    int32_t lanes_per_row;   /* lanes that share one row (1..1024): a power of two, or for the
                                backward with one vector per lane any multiple of 64 up to 1024
                                with wg_threads equal to it (the row is the whole workgroup);
                                split rows: K * 1024 */
    int32_t vecs_per_lane;   /* 16-byte vectors each lane holds per row (vector path) */
    int32_t wg_threads;      /* workgroup size */
    int32_t rows_per_wg;     /* rows a workgroup works on at once */
    int32_t prefetch;        /* row blocks whose loads are issued before the current block's
                                arithmetic. copy_mode 0 (a register ring): 0 or 1; the backward
                                also 2 for one vector per lane (vector path). copy_mode 1: the
                                LDS stages, 2 to 8 */
    int32_t stream_loads;    /* forward, rows of 64 lanes or more: 1 when the row loads carry the
                                non-temporal hint (the ladder sets it; an explicit 0 suits inputs
                                that are still cache-resident); ignored by the backward */
    int32_t elems_per_access; /* element kernels: consecutive elements each access moves (1, 2,
                                4 or 8; at most 16 bytes of activations or weights), dividing N,
                                every pointer aligned to its access; vecs_per_lane *
                                elems_per_access is at most 16 and covers N / 1024. The ladder
                                takes the largest; 0 in an explicit element configuration asks
                                for that one. 0 on the other paths */
    int32_t copy_mode;       /* two-pass forward (vector_path 5): 1 holds 8 vectors per lane
                                after the kept ones in LDS (128 KiB) between the passes, 0
                                none. Backward, vector path, one vector per lane: how the row
                                blocks ahead arrive. 0: loaded into registers (the register ring);
                                1: copied global->LDS by 16-byte direct-to-LDS loads into a ring
                                of `prefetch` LDS stages ("What a tuned RMSNorm kernel actually
                                costs on Hopper", sections 06 and 09: the copy path and the
                                pipeline depth as search dimensions). Built for rows of 256
                                lanes on 1024-lane workgroups (2-4 stages), 512 lanes (2, 3, 4,
                                6, 8), 1024 lanes (2-4) and whole-wavefront rows on the
                                workgroup (2-4); with the fused residual add 2-3 stages (512
                                lanes: 2, 3, 4, 6). 0 on every other path */
    int32_t kept_vecs;       /* two-pass forward (vector_path 5): vectors per lane kept in
                                registers from the first pass for the second, a multiple of
                                vecs_per_lane. Built as (vecs_per_lane, kept_vecs, copy_mode):
                                16-bit (4, 0, 0), (8, 0, 0), (16, 0, 0), (4, 16, 0), (4, 12, 0),
                                (2, 16, 1), (4, 16, 1), (4, 12, 1), residual (4, 0, 0),
                                (8, 0, 0), (2, 16, 0), (4, 12, 0), (2, 16, 1), (4, 12, 1); fp32
                                (4, 0, 0), (8, 0, 0), (16, 0, 0), (2, 14, 0), (4, 12, 0),
                                (2, 14, 1), residual (4, 0, 0), (8, 0, 0), (2, 12, 0), (4, 8, 0),
                                (2, 12, 1); 16-bit with fp32 weights (4, 0, 0), (8, 0, 0),
                                (2, 14, 0), (2, 10, 1), residual (4, 0, 0), (8, 0, 0), (4, 8, 0),
                                (4, 8, 1). 0 on every other path */
    int64_t grid;            /* workgroups launched */
    int64_t partial_rows;    /* backward: fp32 dW partial rows in the workspace (= grid; split
                                rows: grid / K, one per group of K workgroups) */
    int64_t partial_stride;  /* backward: floats between consecutive partial rows */
} rmsnorm_config;

/*
 * Forward. x: [M][N] input; w: [N] weight; y: [M][N] output (same dtype);
 * rstd: [M] fp32 output, or NULL when the caller does not need it.
 * eps must be finite and >= 0 (eps == 0 gives inf/NaN on an all-zero row).
 */
int rmsnorm_fwd(const void *x, const void *w, float eps, int64_t M, int64_t N, int dtype,
                void *y, float *rstd, void *stream);

/*
 * Size in bytes of the fp32 workspace rmsnorm_bwd needs for this shape on the
 * current device (the per-workgroup dW partial rows), or a negative
 * rmsn_status. 0 when M == 0.
 */
int64_t rmsnorm_bwd_workspace_bytes(int64_t M, int64_t N, int dtype);

/*
 * Backward. x, dy: [M][N] (dtype); w: [N] (dtype); rstd: [M] fp32 as written
 * by rmsnorm_fwd for the same x and eps. Outputs: dx [M][N] (dtype) and
 * dW [N] fp32 (overwritten, not accumulated). workspace: device memory of at
 * least rmsnorm_bwd_workspace_bytes(M, N, dtype) bytes, 256-byte aligned; its
 * contents on entry do not matter. Enqueues two kernels on `stream`: the
 * persistent row kernel (dx and per-workgroup dW partials) and a fixed-order
 * combine of the partials ("RMSNorm backward (almost) without the column
 * reduction", section "The persistent kernel"). When the row kernel runs as a
 * single workgroup (a few rows) and dW is 16-byte aligned, that workgroup's
 * partial row is dW and only the row kernel is enqueued. With M == 0, dW is
 * still written (zeros) when N >= 1 and dW is not NULL. dW's summation order
 * depends only on (M, N, dtype), the pointers' alignment class and the
 * device, so the same call gives the same bits every time; each lane's running sums over its
 * rows are fp32 blocks of 8 rows folded into fp64 totals in the register
 * kernels that have room for them (plain fp32 in the others), and the
 * partial rows are added in fp64 and rounded once.
 */
int rmsnorm_bwd(const void *x, const void *w, const void *dy, const float *rstd, int64_t M,
                int64_t N, int dtype, void *dx, float *dw, void *workspace,
                size_t workspace_bytes, void *stream);

/*
 * Fused residual add + RMSNorm (page "Profiling, GPU utilisation and writing
 * a fused kernel", Problem 15: the residual sum and its normalisation
 * produced by one kernel, in one pass over the rows).
 *
 * rmsnorm_fwd_residual: h = x + res rounded to the activation format and
 * stored ([M][N], the residual stream for the next layer); y and rstd are the
 * forward of h as stored, i.e. exactly the unfused add followed by
 * rmsnorm_fwd(h). h must not alias x or res.
 *
 * rmsnorm_bwd_residual: the backward of that pair. h: the stored sum the
 * forward wrote (in place of x); dy: gradient of y; dh: gradient flowing into
 * h from the residual branch. dx = dh + (the rmsnorm input gradient at h),
 * rounded once: the gradient of both x and res. dW as in rmsnorm_bwd. The
 * workspace contract is rmsnorm_bwd's (rmsnorm_bwd_workspace_bytes covers
 * both).
 *
 * cfg: NULL for the ladder's choice, or an explicit configuration as for the
 * *_with_config calls. Same errors as rmsnorm_fwd / rmsnorm_bwd; res / dh must
 * not be NULL when M > 0.
 */
int rmsnorm_fwd_residual(const void *x, const void *res, const void *w, float eps, int64_t M, int64_t N,
                         int dtype, void *h, void *y, float *rstd, const rmsnorm_config *cfg, void *stream);
int rmsnorm_bwd_residual(const void *h, const void *w, const void *dy, const void *dh, const float *rstd,
                         int64_t M, int64_t N, int dtype, void *dx, float *dw, void *workspace,
                         size_t workspace_bytes, const rmsnorm_config *cfg, void *stream);

/*
 * The two kernels of rmsnorm_bwd as separate calls, for callers that time or
 * schedule them apart. rmsnorm_bwd_rows runs the persistent row kernel: dx,
 * and one fp32 partial dW row per workgroup (per group of K workgroups on
 * split rows) in the workspace (rows of round_up(N, 64) floats);
 * *partial_rows receives how many (0 when M == 0).
 * rmsnorm_bwd_combine then writes dW[j] = sum over p < partial_rows of
 * partial[p][j], added in fp64 in an order fixed by (partial_rows, N) and
 * rounded once to fp32. Same arguments,
 * checks and workspace contract as rmsnorm_bwd; rmsnorm_bwd(...) equals rows
 * followed by combine.
 */
int rmsnorm_bwd_rows(const void *x, const void *w, const void *dy, const float *rstd, int64_t M,
                     int64_t N, int dtype, void *dx, void *workspace, size_t workspace_bytes,
                     int64_t *partial_rows, void *stream);
int rmsnorm_bwd_combine(const void *workspace, int64_t partial_rows, int64_t N, float *dw, void *stream);

/*
 * Forward / backward with an explicit launch configuration instead of the
 * ladder's choice: vector_path, lanes_per_row, vecs_per_lane, wg_threads
 * (0: the default, the smallest multiple of lanes_per_row that is at least
 * 256), prefetch, copy_mode (backward only) and grid (>= 1) are read; the
 * other fields are derived. For searching the configuration space ("What a tuned RMSNorm
 * kernel actually costs on Hopper", section 06: the memory-path knobs belong
 * in the search space). Returns RMSN_ECONFIG when the configuration does not
 * cover the row or its kernel is not built, or (split rows) when the grid is
 * more workgroups than the current device keeps resident at once, which is
 * the one check that queries the device (occupancy; nothing is launched
 * before it). The backward workspace must hold
 * grid * partial_stride floats (partial_stride = N rounded up to 64); split
 * rows (vector_path 4): (grid / K) * partial_stride floats, then 16 bytes per
 * workgroup rounded up to 256 (the exchange slots, zeroed by the call). dW
 * bits depend on the configuration.
 */
int rmsnorm_fwd_with_config(const void *x, const void *w, float eps, int64_t M, int64_t N, int dtype,
                            void *y, float *rstd, const rmsnorm_config *cfg, void *stream);
int rmsnorm_bwd_with_config(const void *x, const void *w, const void *dy, const float *rstd, int64_t M,
                            int64_t N, int dtype, void *dx, float *dw, void *workspace,
                            size_t workspace_bytes, const rmsnorm_config *cfg, void *stream);

/*
 * Backward without allocation, for callers that cannot allocate device memory
 * or pass a workspace: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc. Same arguments, results and errors as
 * rmsnorm_bwd, minus the workspace: the fp32 dW partial rows go to a static
 * device array of RMSN_NOALLOC_SCRATCH_BYTES (32 MiB) that the library holds on
 * each GPU it runs on until the process ends. The same kernels with the same
 * grid run, so dx and dW equal rmsnorm_bwd's bit for bit. The call allocates
 * nothing and launches what rmsnorm_bwd launches; its first call on a device
 * looks up that device's copy of the array (hipGetSymbolAddress).
 *
 * Limit: the shape's row kernel must need at most RMSN_NOALLOC_SCRATCH_BYTES
 * of workspace (partial_rows * round_up(N, 64) * 4 bytes, plus 16 bytes per
 * workgroup rounded up to 256 on split rows; bf16 4096 x 32768 needs exactly
 * 32 MiB), else RMSN_ESCRATCH is returned before anything is launched. Every
 * call on one GPU shares that GPU's array: calls that overlap in time on one
 * GPU (two streams, two host threads) race on it and their dW is undefined;
 * calls on one stream are ordered and safe. Nothing in the array needs to
 * start at zero: each call's row kernel writes every partial row its combine
 * reads, and on split rows the call zeroes the exchange slots itself (a fill
 * kernel) before the row kernel.
 */
#define RMSN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int rmsnorm_bwd_noalloc(const void *x, const void *w, const void *dy, const float *rstd, int64_t M,
                        int64_t N, int dtype, void *dx, float *dw, void *stream);

/* Static text for a status code ("ok", "invalid argument", ...). Never NULL. */
const char *rmsnorm_status_str(int status);

/*
 * The ladder as a pure host function (no HIP call): the configuration of the
 * plain (not residual-fused) call for (M, N, dtype, direction) on a device
 * with `num_cus` compute units when the chosen kernel fits `blocks_per_cu`
 * workgroups per compute unit. `aligned`: the alignment of the caller's
 * pointers, 1 for 16-byte aligned, 0 for only aligned to their element type,
 * or 2, 4, 8 or 16 for that many bytes. is_bwd: 0 forward, 1 backward.
 * Returns RMSN_OK or RMSN_EINVAL / RMSN_EDTYPE.
 */
int rmsnorm_select_config(int64_t M, int64_t N, int dtype, int is_bwd, int aligned, int num_cus,
                          int blocks_per_cu, rmsnorm_config *out);

/*
 * The configuration rmsnorm_fwd (is_bwd = 0) or rmsnorm_bwd (is_bwd = 1)
 * would use on the current device for 16-byte aligned pointers, including
 * the occupancy-derived grid. Queries the device (HIP calls).
 */
int rmsnorm_query_config(int64_t M, int64_t N, int dtype, int is_bwd, rmsnorm_config *out);

/* Build identification: compiler, target and flags, as a static string. */
const char *rmsnorm_build_info(void);

#ifdef __cplusplus
}
#endif

#endif /* RMSNORM_MI355X_H */
