// rmsn_bwd_f16w32.hip -- backward vector kernels for fp16 activations, fp32 weights:
// the plain kernels on RMSN_LADDER_SHAPES and the residual-fused ones on
// RMSN_LADDER_SHAPES, the wide-row kernels on RMSN_WIDE_SHAPES_16 (rmsn_instances.h),
// and the lookups the host dispatch uses.
#include "rmsn_bwd_kernels.h"
#include "rmsn_bwd_split.h"
#include "rmsn_instances.h"

namespace rmsn {

#define RMSN_ENTRY(L, V, W, P) {L, V, W, P, reinterpret_cast<const void *>(&bwd_vec<f16_t, float, false, L, V, W, P>)},
static const KernelEntry kPlain[] = {RMSN_LADDER_SHAPES(RMSN_ENTRY) RMSN_BWD_DEEP_SHAPES(RMSN_ENTRY) RMSN_BWD_ROWWG_SHAPES(RMSN_ENTRY)};
#undef RMSN_ENTRY
#define RMSN_ENTRY(L, V, W, P) {L, V, W, P, reinterpret_cast<const void *>(&bwd_vec<f16_t, float, true, L, V, W, P>)},
static const KernelEntry kResidual[] = {RMSN_LADDER_SHAPES(RMSN_ENTRY) RMSN_BWD_DEEP_SHAPES(RMSN_ENTRY) RMSN_BWD_ROWWG_SHAPES(RMSN_ENTRY)};
#undef RMSN_ENTRY

#define RMSN_WIDE_ENTRY(V, P) {kWideLanes, V, kWideLanes, P, reinterpret_cast<const void *>(&bwd_wide<f16_t, float, false, V, (P != 0)>)},
static const KernelEntry kWide[] = {RMSN_WIDE_SHAPES_16(RMSN_WIDE_ENTRY)};
#undef RMSN_WIDE_ENTRY
#define RMSN_WIDE_ENTRY(V, P) {kWideLanes, V, kWideLanes, P, reinterpret_cast<const void *>(&bwd_wide<f16_t, float, true, V, (P != 0)>)},
static const KernelEntry kWideResidual[] = {RMSN_WIDE_SHAPES_16(RMSN_WIDE_ENTRY)};
#undef RMSN_WIDE_ENTRY

const KernelEntry *bwd_vec_kernel_f16w32(int res, int lpr, int vpt, int wg, int pf) {
    return res ? find_entry(kResidual, lpr, vpt, wg, pf) : find_entry(kPlain, lpr, vpt, wg, pf);
}

const KernelEntry *bwd_wide_kernel_f16w32(int res, int vpt, int pf) {
    return find_entry(res ? kWideResidual : kWide, kWideLanes, vpt, kWideLanes, pf);
}
#define RMSN_SPLIT_ENTRY(V, P) {kWideLanes, V, kWideLanes, P, reinterpret_cast<const void *>(&bwd_split<f16_t, float, false, V, (P != 0)>)},
static const KernelEntry kSplit[] = {RMSN_SPLIT_SHAPES_W32(RMSN_SPLIT_ENTRY)};
#undef RMSN_SPLIT_ENTRY
#define RMSN_SPLIT_ENTRY(V, P) {kWideLanes, V, kWideLanes, P, reinterpret_cast<const void *>(&bwd_split<f16_t, float, true, V, (P != 0)>)},
static const KernelEntry kSplitResidual[] = {RMSN_SPLIT_SHAPES_W32(RMSN_SPLIT_ENTRY)};
#undef RMSN_SPLIT_ENTRY

const KernelEntry *bwd_split_kernel_f16w32(int res, int vpt, int pf) {
    return find_entry(res ? kSplitResidual : kSplit, kWideLanes, vpt, kWideLanes, pf);
}

}  // namespace rmsn
