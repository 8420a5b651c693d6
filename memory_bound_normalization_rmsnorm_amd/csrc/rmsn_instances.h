// rmsn_instances.h -- the (lanes per row, vectors per lane, workgroup size,
// prefetch) shapes the vector kernels are built for, as X-macro lists that
// expand X(L, V, W, P) once per shape.
// RMSN_ALL_SHAPES (204 shapes; the fp32 and bf16 kernels, the configuration
// search space):
//   * narrow rows (1..32 lanes, one vector each): 256-lane workgroups;
//   * one or more wavefronts per row with 1..8 vectors per lane, and
//     workgroups of 256, 512 or 1024 lanes (the ladder's default is the
//     smallest that holds a row and four wavefronts);
//   * every shape with and without the register prefetch of the next row.
// RMSN_LADDER_SHAPES (98 shapes; fp16, fp32-weight and residual-fused
// kernels): the same, with only the workgroups the ladder picks per width
// (the row's own, and 1024 lanes for backward rows of 64 to 256 lanes).
#pragma once

#define RMSN_V8(X, L, W, P) X(L, 1, W, P) X(L, 2, W, P) X(L, 3, W, P) X(L, 4, W, P) \
    X(L, 5, W, P) X(L, 6, W, P) X(L, 7, W, P) X(L, 8, W, P)
#define RMSN_PF(M, X, L, W) M(X, L, W, 0) M(X, L, W, 1)
#define RMSN_NARROW(X, L, W, P) X(L, 1, W, P)

#define RMSN_ALL_SHAPES(X)                                                                    \
    RMSN_PF(RMSN_NARROW, X, 1, 256) RMSN_PF(RMSN_NARROW, X, 2, 256)                           \
    RMSN_PF(RMSN_NARROW, X, 4, 256) RMSN_PF(RMSN_NARROW, X, 8, 256)                           \
    RMSN_PF(RMSN_NARROW, X, 16, 256) RMSN_PF(RMSN_NARROW, X, 32, 256)                         \
    RMSN_PF(RMSN_V8, X, 64, 256) RMSN_PF(RMSN_V8, X, 64, 512) RMSN_PF(RMSN_V8, X, 64, 1024)    \
    RMSN_PF(RMSN_V8, X, 128, 256) RMSN_PF(RMSN_V8, X, 128, 512) RMSN_PF(RMSN_V8, X, 128, 1024) \
    RMSN_PF(RMSN_V8, X, 256, 256) RMSN_PF(RMSN_V8, X, 256, 512) RMSN_PF(RMSN_V8, X, 256, 1024) \
    RMSN_PF(RMSN_V8, X, 512, 512) RMSN_PF(RMSN_V8, X, 512, 1024)                              \
    RMSN_PF(RMSN_V8, X, 1024, 1024)

#define RMSN_LADDER_SHAPES(X)                                                                 \
    RMSN_PF(RMSN_NARROW, X, 1, 256) RMSN_PF(RMSN_NARROW, X, 2, 256)                           \
    RMSN_PF(RMSN_NARROW, X, 4, 256) RMSN_PF(RMSN_NARROW, X, 8, 256)                           \
    RMSN_PF(RMSN_NARROW, X, 16, 256) RMSN_PF(RMSN_NARROW, X, 32, 256)                         \
    RMSN_PF(RMSN_V8, X, 64, 256) RMSN_PF(RMSN_V8, X, 128, 256) RMSN_PF(RMSN_V8, X, 256, 256)  \
    RMSN_PF(RMSN_NARROW, X, 64, 1024) RMSN_PF(RMSN_NARROW, X, 128, 1024)                      \
    RMSN_PF(RMSN_NARROW, X, 256, 1024)                                                        \
    RMSN_PF(RMSN_V8, X, 512, 512) RMSN_PF(RMSN_V8, X, 1024, 1024)

// Wide-row backward kernels (1024 lanes, dW sums in LDS), as (vectors per
// lane, prefetch): at most 128 KiB of sums, i.e. 4 vectors of 8 16-bit
// elements or 8 vectors of 4 fp32 elements per lane. fp32 rows of 6 or more
// vectors per lane have no prefetching variant (it does not fit in 128 VGPRs).
#define RMSN_WIDE_SHAPES_16(X) X(2, 0) X(2, 1) X(3, 0) X(3, 1) X(4, 0) X(4, 1)
#define RMSN_WIDE_SHAPES_32(X) X(2, 0) X(2, 1) X(3, 0) X(3, 1) X(4, 0) X(4, 1) X(5, 0) X(5, 1) \
    X(6, 0) X(7, 0) X(8, 0)

// Backward kernels with two row blocks prefetched (depth 2), for the shapes the
// backward ladder uses with one vector per lane.
#define RMSN_BWD_DEEP_SHAPES(X) X(1, 1, 256, 2) X(2, 1, 256, 2) X(4, 1, 256, 2) X(8, 1, 256, 2) \
    X(16, 1, 256, 2) X(32, 1, 256, 2) X(64, 1, 1024, 2) X(128, 1, 1024, 2) X(256, 1, 1024, 2)   \
    X(512, 1, 512, 2) X(1024, 1, 1024, 2)

// Backward kernels whose row is the whole workgroup, sized at launch to the
// row's vectors rounded up to whole wavefronts (one vector per lane), for
// rows of 256 to 1024 vectors that are not a power of two (640 lanes at 5120
// 16-bit columns instead of 1024 with 3/8 idle), as (0, 1, launch bound,
// prefetch depth).
#define RMSN_BWD_ROWWG_SHAPES(X) X(0, 1, 1024, 1) X(0, 1, 1024, 2)

// LDS-staged backward kernels (rmsn_bwd_lds.h), as (lanes per row, workgroup,
// stages): rows of 256 lanes on 1024-lane workgroups, rows of 512 and 1024
// lanes, and rows on whole wavefronts sized at launch (0), each with the
// stage counts that fit in 160 KiB of LDS (three inputs per stage with the
// fused residual add).
#define RMSN_LDS_SHAPES(X) X(256, 1024, 2) X(256, 1024, 3) X(256, 1024, 4)                             \
    X(512, 512, 2) X(512, 512, 3) X(512, 512, 4) X(512, 512, 6) X(512, 512, 8)                          \
    X(1024, 1024, 2) X(1024, 1024, 3) X(1024, 1024, 4) X(0, 1024, 2) X(0, 1024, 3) X(0, 1024, 4)
#define RMSN_LDS_RES_SHAPES(X) X(256, 1024, 2) X(256, 1024, 3) X(512, 512, 2) X(512, 512, 3)            \
    X(512, 512, 4) X(512, 512, 6) X(1024, 1024, 2) X(1024, 1024, 3) X(0, 1024, 2) X(0, 1024, 3)

// Wide-row backward kernels with the next row staged through LDS
// (rmsn_bwd_lds.h bwd_wide_lds; 16-bit activations only), as (lanes per row,
// vectors per lane, stages): a whole row of x and dy per stage, so one stage
// at 24576 columns and up to two at 16384; 1024 lanes at 2 and 3 vectors per
// lane, 512 lanes (256 registers per lane) at 4 and 6. Rows of 32768 columns
// have none: at 8 vectors per lane on 512 lanes the dW sums and the row spill
// (bf16: 269 us against 149 for bwd_wide at 4096 x 32768).
#define RMSN_WIDE_LDS_SHAPES(X) X(1024, 2, 1) X(1024, 2, 2) X(1024, 3, 1) X(512, 4, 1) X(512, 4, 2) \
    X(512, 6, 1)

// Forward rows of 8193 to 16384 16-byte vectors (131072 16-bit or 65536
// fp32 columns) on one 1024-lane workgroup, 9 to 16 vectors per lane (the
// weights re-read from cache), plain forward only.
#define RMSN_FWD_XWIDE_SHAPES(X) X(1024, 9, 1024, 0) X(1024, 10, 1024, 0) X(1024, 11, 1024, 0) \
    X(1024, 12, 1024, 0) X(1024, 13, 1024, 0) X(1024, 14, 1024, 0) X(1024, 15, 1024, 0) X(1024, 16, 1024, 0)

// Forward rows beyond what the vector kernels hold in registers (more than
// 16 vectors per lane on 1024 lanes, 8 with the residual add): the two-pass
// kernel (rmsn_fwd_loop.h), as (vectors per lane per chunk, waves per SIMD:
// 8 for two workgroups per CU, 4 for one, vectors per lane kept in registers
// between the passes, vectors per lane held in LDS after those), per format
// (16-bit, fp32, 16-bit with fp32 weights), plain and residual-fused. The
// kept vectors are the most each format holds without spilling at one
// workgroup per CU; the held ones fill 128 KiB of LDS. The shapes that keep
// none run two per CU wherever the kernel fits 64 VGPRs.
#define RMSN_FWD_LOOP_SHAPES_16(X) X(4, 8, 0, 0) X(8, 8, 0, 0) X(16, 4, 0, 0) X(4, 4, 16, 0) X(4, 4, 12, 0) \
    X(2, 4, 16, 8) X(4, 4, 16, 8) X(4, 4, 12, 8)
#define RMSN_FWD_LOOP_SHAPES_32(X) X(4, 8, 0, 0) X(8, 4, 0, 0) X(16, 4, 0, 0) X(2, 4, 14, 0) X(4, 4, 12, 0) \
    X(2, 4, 14, 8)
#define RMSN_FWD_LOOP_SHAPES_W32(X) X(4, 8, 0, 0) X(8, 8, 0, 0) X(2, 4, 14, 0) X(2, 4, 10, 8)
#define RMSN_FWD_LOOP_RES_SHAPES_16(X) X(4, 8, 0, 0) X(8, 4, 0, 0) X(2, 4, 16, 0) X(4, 4, 12, 0) X(2, 4, 16, 8) \
    X(4, 4, 12, 8)
#define RMSN_FWD_LOOP_RES_SHAPES_32(X) X(4, 8, 0, 0) X(8, 4, 0, 0) X(2, 4, 12, 0) X(4, 4, 8, 0) X(2, 4, 12, 8)
#define RMSN_FWD_LOOP_RES_SHAPES_W32(X) X(4, 4, 0, 0) X(8, 4, 0, 0) X(4, 4, 8, 0) X(4, 4, 8, 8)

// Backward rows split over K workgroups (rmsn_bwd_split.h), as (vectors per
// lane, prefetch). Two workgroups per CU: 2 vectors per lane of 16-bit
// activations (the ladder's choice up to 16 members); one per CU: 3-4
// (16-bit) or 5-8 (fp32) for wider rows, fp32 rows and the configuration
// search. Prefetch with 16-bit weights at one per CU only (at two it spills).
#define RMSN_SPLIT_SHAPES_16(X) X(2, 0) X(3, 0) X(3, 1) X(4, 0) X(4, 1)
#define RMSN_SPLIT_SHAPES_W32(X) X(2, 0) X(3, 0) X(4, 0)
#define RMSN_SPLIT_SHAPES_32(X) X(5, 0) X(6, 0) X(7, 0) X(8, 0)

namespace rmsn {

template <int N>
const KernelEntry *find_entry(const KernelEntry (&t)[N], int lpr, int vpt, int wg, int pf) {
    for (int i = 0; i < N; ++i)
        if (t[i].lpr == lpr && t[i].vpt == vpt && t[i].wg == wg && t[i].pf == pf) return &t[i];
    return nullptr;
}

}  // namespace rmsn
