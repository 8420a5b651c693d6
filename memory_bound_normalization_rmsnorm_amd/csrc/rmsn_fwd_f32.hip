// rmsn_fwd_f32.hip -- forward vector kernels for fp32 activations and weights:
// the plain kernels on RMSN_ALL_SHAPES and RMSN_FWD_XWIDE_SHAPES, the
// residual-fused ones on RMSN_LADDER_SHAPES (rmsn_instances.h), the two-pass
// kernels for wider rows on RMSN_FWD_LOOP_SHAPES_32 and
// RMSN_FWD_LOOP_RES_SHAPES_32, and the lookups the host dispatch uses.
#include "rmsn_fwd_kernels.h"
#include "rmsn_fwd_loop.h"
#include "rmsn_instances.h"

namespace rmsn {

#define RMSN_ENTRY(L, V, W, P) {L, V, W, P, reinterpret_cast<const void *>(&fwd_vec<float, float, false, L, V, W, (P != 0)>)},
static const KernelEntry kPlain[] = {RMSN_ALL_SHAPES(RMSN_ENTRY) RMSN_FWD_XWIDE_SHAPES(RMSN_ENTRY)};
#undef RMSN_ENTRY
#define RMSN_ENTRY(L, V, W, P) {L, V, W, P, reinterpret_cast<const void *>(&fwd_vec<float, float, true, L, V, W, (P != 0)>)},
static const KernelEntry kResidual[] = {RMSN_LADDER_SHAPES(RMSN_ENTRY)};
#undef RMSN_ENTRY

const KernelEntry *fwd_vec_kernel_f32(int res, int lpr, int vpt, int wg, int pf) {
    return res ? find_entry(kResidual, lpr, vpt, wg, pf) : find_entry(kPlain, lpr, vpt, wg, pf);
}

#define RMSN_LOOP_ENTRY(C, W, K, L) {kWideLanes, C, kWideLanes, W, reinterpret_cast<const void *>(&fwd_loop<float, float, false, C, W, K, L>), K, L},
static const KernelEntry kLoop[] = {RMSN_FWD_LOOP_SHAPES_32(RMSN_LOOP_ENTRY)};
#undef RMSN_LOOP_ENTRY
#define RMSN_LOOP_ENTRY(C, W, K, L) {kWideLanes, C, kWideLanes, W, reinterpret_cast<const void *>(&fwd_loop<float, float, true, C, W, K, L>), K, L},
static const KernelEntry kLoopResidual[] = {RMSN_FWD_LOOP_RES_SHAPES_32(RMSN_LOOP_ENTRY)};
#undef RMSN_LOOP_ENTRY

// the two-pass kernel of `ch` vectors per lane per chunk, `kv` of them kept in
// registers between the passes and the next `lv` held in LDS (its waves per
// SIMD in the entry's prefetch field)
const KernelEntry *fwd_loop_kernel_f32(int res, int ch, int kv, int lv) {
    const KernelEntry *t = res ? kLoopResidual : kLoop;
    const int n = res ? (int)(sizeof kLoopResidual / sizeof *kLoopResidual) : (int)(sizeof kLoop / sizeof *kLoop);
    for (int i = 0; i < n; ++i)
        if (t[i].vpt == ch && t[i].kv == kv && t[i].lv == lv) return &t[i];
    return nullptr;
}

}  // namespace rmsn
