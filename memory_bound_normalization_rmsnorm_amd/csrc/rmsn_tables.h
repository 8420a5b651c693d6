// rmsn_tables.h -- kernel lookup shared by the kernel files and the host API.
#pragma once

#include <stdint.h>

namespace rmsn {

// Lanes of the scalar (any-N, any-alignment) row kernels and the combine kernel.
constexpr int kScalarWG = 256;
constexpr int kScalarLdsCols = 16384;  // scalar backward rows up to this width keep their dW sums in LDS (64 KiB)
// Element kernels (rows that are not a multiple of 16 bytes or not 16-byte
// aligned): kElemMinLanes to kElemMaxLanes lanes per row (a power of two), at
// most kElemMaxK elements per lane.
constexpr int kElemMinLanes = 64;
constexpr int kElemMaxLanes = 1024;
constexpr int kElemMaxK = 16;
constexpr int kCombineWG = 512;
constexpr int kCombineUnroll = 8;    // partial-row loads a combine lane has in flight
constexpr int kPartialAlign = 64;    // partial rows are padded to a multiple of 64 floats

// Workgroup size for a row group of `lpr` lanes: at least four wavefronts.
constexpr int wg_for_lpr(int lpr) { return lpr > 256 ? lpr : 256; }

// Waves per SIMD the compiler is asked to fit (512 VGPRs per SIMD lane), from
// the registers a lane needs with rows and weights kept packed: `packed`
// 16-byte vectors (4 VGPRs each), `floats` fp32 accumulators, one offset per
// vector and 24 + `extra` temporaries (the unpacked operands of one vector:
// kernels that combine more inputs per element pass more). The scheduler then
// trades ILP for occupancy instead of unpacking every operand ahead of use.
// A workgroup of `wg` lanes occupies wg/256 waves on each of the 4 SIMDs, so
// never ask for fewer than that.
constexpr int waves_for(int packed, int floats, int vpt, int wg, int extra = 0) {
    const int regs = 4 * packed + floats + vpt + 24 + extra;
    int w = 512 / regs;
    const int need = wg / 256 > 1 ? wg / 256 : 1;
    w = w < need ? need : w;
    return w > 8 ? 8 : w;
}

// Wide-row backward kernels: 1024 lanes per row, dW sums in LDS (at most
// 128 KiB of the CU's 160 KiB).
constexpr int kWideLanes = 1024;
constexpr int kWideLdsBytes = 128 * 1024;

struct KernelEntry {
    int lpr;         // lanes per row
    int vpt;         // 16-byte vectors per lane
    int wg;          // workgroup size
    int pf;          // 1: next row's loads issued before the current row's arithmetic
    const void *fn;  // __global__ function
    int kv = 0;      // two-pass forward: vectors per lane kept in registers between the passes
    int lv = 0;      // two-pass forward: vectors per lane held in LDS after the kept ones
};

// dtype: an rmsn_dtype code (activation and weight formats); res: 1 for the
// residual-fused kernels. nullptr when (lpr, vpt, wg, pf) is not instantiated.
const KernelEntry *fwd_vec_kernel(int dtype, int res, int lpr, int vpt, int wg, int pf);
const KernelEntry *bwd_vec_kernel(int dtype, int res, int lpr, int vpt, int wg, int pf);
// wide-row backward kernels (lanes per row and workgroup kWideLanes)
const KernelEntry *bwd_wide_kernel(int dtype, int res, int vpt, int pf);
// LDS-staged backward kernels (one vector per lane): rows of `lpr` lanes (0:
// the whole workgroup, sized at launch) on `wg`-lane workgroups, `st` row
// blocks in flight; KernelEntry::pf holds st
const KernelEntry *bwd_lds_kernel(int dtype, int res, int lpr, int wg, int st);
// wide-row backward kernels (`lpr` = 512 or 1024 lanes, `vpt` vectors per lane)
// with the next `st` rows staged through LDS; plain (not residual) 16-bit activations
const KernelEntry *bwd_wide_lds_kernel(int dtype, int lpr, int vpt, int st);
// backward rows split over several 1024-lane workgroups (rmsn_bwd_split.h),
// `vpt` vectors per lane of the workgroup's slice
const KernelEntry *bwd_split_kernel(int dtype, int res, int vpt, int pf);
// forward rows beyond the vector kernels: the two-pass kernel of `ch` vectors
// per lane per chunk, `kv` of them kept in registers and the next `lv` held
// in LDS (rmsn_fwd_loop.h)
const KernelEntry *fwd_loop_kernel(int dtype, int res, int ch, int kv, int lv);
// bytes of one workgroup's exchange slot of the split backward
constexpr int kSplitSlotBytes = 16;
// most workgroups a split row may take
constexpr int kMaxSplit = 16;
// lds: the backward kernel that keeps its dW sums in LDS (rows of at most kScalarLdsCols columns)
const void *scalar_kernel(int dtype, int is_bwd, int res, int lds);
// element kernels: rows of `lanes` lanes (64, 128, 256, 512 or 1024), k
// accesses of g elements per lane (g 1, 2, 4 or 8, at most 16 bytes per
// access; k * g at most kElemMaxK), nullptr otherwise
const void *elem_kernel(int dtype, int is_bwd, int res, int k, int g, int lanes);
// the fixed-order dW combine summing `slices` (8, 16, 32 or 64) partial rows
// side by side, 4 * kCombineWG / slices columns per workgroup; nullptr otherwise
const void *dw_combine_kernel(int slices);
const void *fill_zero_kernel();

// Device address of the current device `dev`'s copy of the static workspace
// of rmsnorm_bwd_noalloc (RMSN_NOALLOC_SCRATCH_BYTES, 256-byte aligned),
// looked up on the first call per device and cached. RMSN_OK or RMSN_EHIP.
int scratch_region(int dev, void **ptr);

}  // namespace rmsn
