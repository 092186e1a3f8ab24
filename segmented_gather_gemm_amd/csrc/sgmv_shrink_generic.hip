// Generic LoRA-A projection (shrink) kernels: any shape, stride and
// alignment.  Device code and design notes: sgmv_shrink.h.
#include "sgmv_shrink.h"

namespace sgmv {
namespace dev {

template <int XD, int WD>
const void* shrink_generic_by_out(int od) {
  switch (od) {
    case F16: return reinterpret_cast<const void*>(&shrink_generic<XD, WD, F16>);
    case BF16: return reinterpret_cast<const void*>(&shrink_generic<XD, WD, BF16>);
    case F32: return reinterpret_cast<const void*>(&shrink_generic<XD, WD, F32>);
    default: return nullptr;
  }
}

inline const void* shrink_generic_table(int xd, int wd, int od) {
  if (wd == BF16 && xd == BF16) return shrink_generic_by_out<BF16, BF16>(od);
  if (wd == BF16 && xd == F32) return shrink_generic_by_out<F32, BF16>(od);
  if (wd == F16 && xd == F16) return shrink_generic_by_out<F16, F16>(od);
  if (wd == F16 && xd == F32) return shrink_generic_by_out<F32, F16>(od);
  return nullptr;
}

}  // namespace dev

const void* shrink_generic_kernel(int xd, int wd, int od) {
  return dev::shrink_generic_table(xd, wd, od);
}

}  // namespace sgmv
