// Fused LoRA delta kernels (shrink and expand in one launch) for ranks of
// 2 k tile(s) of 16 rows per slice.  Device code and design notes:
// sgmv_fused.h.
#include "sgmv_fused.h"

namespace sgmv {

const void* fused_kernel_k2(int xd, int wd, int od, bool add, int ns, bool split_h) {
  return dev::fused_table<2>(xd, wd, od, add, ns, split_h);
}

}  // namespace sgmv
