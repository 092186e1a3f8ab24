// Generic SGMV expand-slice kernels: any rank, shape, stride and alignment.
// Device code and design notes: sgmv_device.h.
#include "sgmv_device.h"

namespace sgmv {

const void* generic_kernel(int xd, int wd, int od, bool add) {
  return dev::generic_table(xd, wd, od, add);
}

}  // namespace sgmv
