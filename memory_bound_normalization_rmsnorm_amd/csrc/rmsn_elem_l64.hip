// rmsn_elem_l64.hip -- the element kernels with 64 lanes per row (each lane
// count in its own translation unit, so that they compile in parallel).
#include "rmsn_elem_kernels.h"

namespace rmsn {

template const void *elem_pick<64>(int, int, int, int, int);

}  // namespace rmsn
