// Fast SGMV expand-slice kernels for ranks up to 64 (rank steps = 2).
// Device code and design notes: sgmv_device.h.
#include "sgmv_device.h"

namespace sgmv {

const void* fast_kernel_ks2(int xd, int wd, int od, bool add, bool gather) {
  return dev::fast_table<2>(xd, wd, od, add, gather);
}

}  // namespace sgmv
