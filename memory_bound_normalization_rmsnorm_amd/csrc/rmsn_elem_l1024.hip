// rmsn_elem_l1024.hip -- the element kernels with 1024 lanes per row (each lane
// count in its own translation unit, so that they compile in parallel).
#include "rmsn_elem_kernels.h"

namespace rmsn {

template const void *elem_pick<1024>(int, int, int, int, int);

const void *elem_kernel(int dtype, int is_bwd, int res, int k, int g, int lanes) {
    switch (lanes) {
    case 64: return elem_pick<64>(dtype, is_bwd, res, k, g);
    case 128: return elem_pick<128>(dtype, is_bwd, res, k, g);
    case 256: return elem_pick<256>(dtype, is_bwd, res, k, g);
    case 512: return elem_pick<512>(dtype, is_bwd, res, k, g);
    case 1024: return elem_pick<1024>(dtype, is_bwd, res, k, g);
    default: return nullptr;
    }
}

}  // namespace rmsn
