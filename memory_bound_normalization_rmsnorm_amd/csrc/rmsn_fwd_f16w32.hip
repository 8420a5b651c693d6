// rmsn_fwd_f16w32.hip -- forward vector kernels for fp16 activations, fp32 weights:
// the plain kernels on RMSN_LADDER_SHAPES and RMSN_FWD_XWIDE_SHAPES, the residual-fused ones on
// RMSN_LADDER_SHAPES (rmsn_instances.h), and the lookup the host dispatch uses.
#include "rmsn_fwd_kernels.h"
#include "rmsn_instances.h"

namespace rmsn {

#define RMSN_ENTRY(L, V, W, P) {L, V, W, P, reinterpret_cast<const void *>(&fwd_vec<f16_t, float, false, L, V, W, (P != 0)>)},
static const KernelEntry kPlain[] = {RMSN_LADDER_SHAPES(RMSN_ENTRY) RMSN_FWD_XWIDE_SHAPES(RMSN_ENTRY)};
#undef RMSN_ENTRY
#define RMSN_ENTRY(L, V, W, P) {L, V, W, P, reinterpret_cast<const void *>(&fwd_vec<f16_t, float, true, L, V, W, (P != 0)>)},
static const KernelEntry kResidual[] = {RMSN_LADDER_SHAPES(RMSN_ENTRY)};
#undef RMSN_ENTRY

const KernelEntry *fwd_vec_kernel_f16w32(int res, int lpr, int vpt, int wg, int pf) {
    return res ? find_entry(kResidual, lpr, vpt, wg, pf) : find_entry(kPlain, lpr, vpt, wg, pf);
}

}  // namespace rmsn
