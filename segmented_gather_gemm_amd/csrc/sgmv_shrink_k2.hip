// Fast LoRA-A projection (shrink) kernels for ranks of 2 k tile(s) of 16
// rows per slice.  Device code and design notes: sgmv_shrink.h.
#include "sgmv_shrink.h"

namespace sgmv {

const void* shrink_kernel_k2(int xd, int wd, int od, int ns, bool split_t) {
  return dev::shrink_table<2>(xd, wd, od, ns, split_t);
}

}  // namespace sgmv
