// sgmv_limits.h -- size predicates of libsgmv's kernel choices and the
// work-assignment arithmetic of its kernels, kept free of HIP headers so
// that they can be checked on any host (the constexpr function below is
// also compiled for the device).  Internal to libsgmv.
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

// The units [begin, end) of U that workgroup `bid` of a grid of G runs (the
// kernels that split their units into contiguous ranges; cus = the device's
// compute units).  With G = 8 k (k >= 2), workgroups i and i' run on the
// same XCD when i = i' mod 8 (round-robin dispatch; measured on MI355X,
// which also places the first 256 workgroups of a launch one per compute
// unit), and each XCD serves one contiguous part of the units:
//  * U <= G and U <= cus (the host sizes the grid from an upper bound of U,
//    so often G > U): XCD x = i % 8 takes the share [x U/8, (x + 1) U/8)
//    (sizes differ by at most one) and gives its units to its workgroups in
//    order of i / 8, so every unit has a compute unit of its own.  Filling
//    XCD after XCD instead left whole XCDs idle and doubled the units on the
//    others' compute units (split-T shrink, 192 units of 64 rows: 63 us
//    against 41);
//  * otherwise workgroups renumbered XCD-major, lw = (i % 8) k + i / 8, take
//    contiguous ranges by lw, the first ones one unit more.  With more units
//    than compute units some of them run two either way; this keeps the
//    extra ones on consecutive units of the first XCDs (adjacent units share
//    an adapter in one L2), measured 1-5% faster than spreading them for the
//    fused kernel (298 units, grid 256) and the shrink (298 units, grid 320).
// Other grids: plain contiguous ranges.  The arithmetic is 32-bit (unit
// counts and indices are below 2^31).
struct UnitSpan {
  uint32_t begin, end;
};
constexpr UnitSpan unit_span(uint32_t U, uint32_t G, uint32_t cus, uint32_t bid) {
  uint32_t base = 0, n = U, m = G, i = bid;
  if (G >= 16 && (G & 7) == 0) {
    if (U <= G && U <= cus) {
      const uint32_t x = bid & 7, share = U >> 3, extra = U & 7;
      base = x * share + (x < extra ? x : extra);
      n = share + (x < extra ? 1u : 0u);
      m = G >> 3;
      i = bid >> 3;
    } else {
      i = (bid & 7) * (G >> 3) + (bid >> 3);
    }
  }
  const uint32_t q = n / m, r = n - q * m;
  const uint32_t b = base + i * q + (i < r ? i : r);
  return UnitSpan{b, b + q + (i < r ? 1u : 0u)};
}

}  // namespace limits
}  // namespace sgmv
