// Fast SGMV expand-slice kernels for ranks up to 16 (one rank step, input
// tile loaded by every wave).  Device code and design notes: sgmv_device.h.
#include "sgmv_device.h"

namespace sgmv {

const void* fast_kernel_ks0(int xd, int wd, int od, bool add, bool gather) {
  return dev::fast_table<0>(xd, wd, od, add, gather);
}

}  // namespace sgmv
