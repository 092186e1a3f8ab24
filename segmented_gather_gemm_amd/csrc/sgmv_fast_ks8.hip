// Fast SGMV expand-slice kernels for ranks up to 256 (rank steps = 8).
// Device code and design notes: sgmv_device.h.
#include "sgmv_device.h"

namespace sgmv {

const void* fast_kernel_ks8(int xd, int wd, int od, bool add, bool gather) {
  return dev::fast_table<8>(xd, wd, od, add, gather);
}

}  // namespace sgmv
