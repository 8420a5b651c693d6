// rmsn_bwd_bf16.hip -- backward vector kernels, bf16 storage: every
// shape of rmsn_instances.h, and the lookup the host dispatch uses.
#include "rmsn_bwd_kernels.h"
#include "rmsn_instances.h"

namespace rmsn {

#define RMSN_ENTRY(L, V, W, P) {L, V, W, P, reinterpret_cast<const void *>(&bwd_vec<bf16_t, L, V, W, (P != 0)>)},
static const KernelEntry kTable[] = {RMSN_ALL_SHAPES(RMSN_ENTRY)};
#undef RMSN_ENTRY

const KernelEntry *bwd_vec_kernel_bf16(int lpr, int vpt, int wg, int pf) { return find_entry(kTable, lpr, vpt, wg, pf); }

}  // namespace rmsn
