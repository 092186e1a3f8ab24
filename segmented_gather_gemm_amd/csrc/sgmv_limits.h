// sgmv_limits.h -- host-side size predicates of libsgmv's kernel choices,
// kept free of HIP headers so that they can be checked on any host.
// Internal to libsgmv.
#pragma once

#include <stdint.h>

namespace sgmv {
namespace limits {

// Smallest power of two >= v (v >= 1).
inline int64_t next_pow2(int64_t v) {
  int64_t p = 1;
  while (p < v) p <<= 1;
  return p;
}

// The fast LoRA-A projection kernels address one adapter's lora_A block
// (rank K rows of H 16-bit elements) with 32-bit buffer offsets over the
// 16 k16 rows their k tiles cover (k16 = next power of two of ceil(K / 16);
// the rows past K lie outside the block's buffer resource and read zero),
// and give masked lanes the offset 2^31, which must lie past the resource.
// Both hold when those rows span less than 2 GiB.
inline bool shrink_fast_lora_a_fits(int64_t K, int64_t H) {
  if (K < 1 || H < 1 || H >= (int64_t(1) << 31)) return false;
  const int64_t rows = 16 * next_pow2((K + 15) / 16);
  return rows * H * 2 < (int64_t(1) << 31);
}

}  // namespace limits
}  // namespace sgmv
