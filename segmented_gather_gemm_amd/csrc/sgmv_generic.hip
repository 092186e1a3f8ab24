// Generic SGMV expand-slice kernels: any rank, shape, stride and alignment.
// Device code and design notes: sgmv_device.h.
#include "sgmv_device.h"

namespace sgmv {
namespace dev {

template <int XD, int WD, int OD>
const void* generic_entry(bool add) {
  return add ? reinterpret_cast<const void*>(&expand_generic<XD, WD, OD, true>)
             : reinterpret_cast<const void*>(&expand_generic<XD, WD, OD, false>);
}

template <int XD, int WD>
const void* generic_by_out(int od, bool add) {
  switch (od) {
    case F16: return generic_entry<XD, WD, F16>(add);
    case BF16: return generic_entry<XD, WD, BF16>(add);
    case F32: return generic_entry<XD, WD, F32>(add);
    default: return nullptr;
  }
}

inline const void* generic_table(int xd, int wd, int od, bool add) {
  if (wd == BF16 && xd == BF16) return generic_by_out<BF16, BF16>(od, add);
  if (wd == BF16 && xd == F32) return generic_by_out<F32, BF16>(od, add);
  if (wd == F16 && xd == F16) return generic_by_out<F16, F16>(od, add);
  if (wd == F16 && xd == F32) return generic_by_out<F32, F16>(od, add);
  return nullptr;
}

}  // namespace dev

const void* generic_kernel(int xd, int wd, int od, bool add) {
  return dev::generic_table(xd, wd, od, add);
}

}  // namespace sgmv
