// Fast LoRA-A projection (shrink) kernels with 16 k tile(s) of 16 rows over
// all slices.  Device code and design notes: sgmv_shrink.h.
#include "sgmv_shrink.h"

namespace sgmv {

const void* shrink_kernel_kt16(int xd, int wd, int od) { return dev::shrink_table<16>(xd, wd, od); }

}  // namespace sgmv
