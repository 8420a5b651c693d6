// rmsn_bwd_lds_bf16.hip -- LDS-staged backward kernels (rmsn_bwd_lds.h) for
// bf16 activations and weights: the plain kernels on RMSN_LDS_SHAPES and the residual-fused
// ones on RMSN_LDS_RES_SHAPES, the wide-row ones on RMSN_WIDE_LDS_SHAPES
// (rmsn_instances.h), and their lookups.
#include "rmsn_bwd_lds.h"
#include "rmsn_instances.h"

namespace rmsn {

#define RMSN_ENTRY(L, W, S) {L, 1, W, S, reinterpret_cast<const void *>(&bwd_lds<bf16_t, bf16_t, false, L, W, S>)},
static const KernelEntry kLds[] = {RMSN_LDS_SHAPES(RMSN_ENTRY)};
#undef RMSN_ENTRY
#define RMSN_ENTRY(L, W, S) {L, 1, W, S, reinterpret_cast<const void *>(&bwd_lds<bf16_t, bf16_t, true, L, W, S>)},
static const KernelEntry kLdsResidual[] = {RMSN_LDS_RES_SHAPES(RMSN_ENTRY)};
#undef RMSN_ENTRY

const KernelEntry *bwd_lds_kernel_bf16(int res, int lpr, int wg, int st) {
    return res ? find_entry(kLdsResidual, lpr, 1, wg, st) : find_entry(kLds, lpr, 1, wg, st);
}

#define RMSN_WIDE_ENTRY(L, V, S) {L, V, L, S, reinterpret_cast<const void *>(&bwd_wide_lds<bf16_t, bf16_t, L, V, S>)},
static const KernelEntry kWideLds[] = {RMSN_WIDE_LDS_SHAPES(RMSN_WIDE_ENTRY)};
#undef RMSN_WIDE_ENTRY

const KernelEntry *bwd_wide_lds_kernel_bf16(int lpr, int vpt, int st) { return find_entry(kWideLds, lpr, vpt, lpr, st); }

}  // namespace rmsn
