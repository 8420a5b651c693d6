// rmsn_fwd_f32.hip -- forward vector kernels, fp32 storage: every
// shape of rmsn_instances.h, and the lookup the host dispatch uses.
#include "rmsn_fwd_kernels.h"
#include "rmsn_instances.h"

namespace rmsn {

#define RMSN_ENTRY(L, V, W, P) {L, V, W, P, reinterpret_cast<const void *>(&fwd_vec<float, L, V, W, (P != 0)>)},
static const KernelEntry kTable[] = {RMSN_ALL_SHAPES(RMSN_ENTRY)};
#undef RMSN_ENTRY

const KernelEntry *fwd_vec_kernel_f32(int lpr, int vpt, int wg, int pf) { return find_entry(kTable, lpr, vpt, wg, pf); }

}  // namespace rmsn
