// sgmv_limits.h -- size predicates of libsgmv's kernel choices and the
// work-assignment arithmetic of its kernels, kept free of HIP headers so
// that they can be checked on any host (the constexpr functions below are
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

// Balanced split-T shrink (calls that bring a workspace).  With C compute
// units (C % 8 == 0) and C < U <= 2 C units of 64 tokens, some compute
// units would run two units where the others run one, and those set the
// time (a unit alone takes ~40 us at hidden 4096, two resident ~52-60).
// Instead workgroups 0..C-1 take one unit each (unit_span over the first C
// units), and the E = U - C other units are cut into P parts over the
// hidden steps, taken by workgroups C, C + 1, ...: part r of unit C + e is
// workgroup C + e P + r.  Parts write fp32 partial sums to the workspace;
// the last part of a unit to finish adds them in part order and stores the
// result, so every compute unit holds about U / C units of work.
// P = min(C / E, kShrinkMaxParts, ceil(h_steps / 4)).  plan.P == 0: the
// call does not qualify (workspace-free launch, U outside (C, 2 C], a grid
// below 2 C, or P < 2: with more than 1.5 C units whole overflow units on
// workgroups C.. measured 4-5% slower than unit_span's XCD-major fill) and
// the units are split by unit_span.
#ifndef SGMV_SHRINK_MAX_PARTS
#define SGMV_SHRINK_MAX_PARTS 4
#endif
constexpr uint32_t kShrinkMaxParts = SGMV_SHRINK_MAX_PARTS;
// Workspace bytes of one part's partial sums: 64 tokens x 256 rows (16 k
// tiles, the most one launch takes) of fp32.
constexpr uint32_t kShrinkPartBytes = 64u * 256u * 4u;

struct PartPlan {
  uint32_t E, P;  // overflow units, parts per overflow unit
};
constexpr PartPlan part_plan(uint32_t U, uint32_t C, uint32_t G, uint32_t h_steps) {
  if (C < 8 || (C & 7) != 0 || U <= C || U > 2 * C || G < 2 * C || h_steps == 0)
    return PartPlan{0, 0};
  const uint32_t E = U - C, n4 = (h_steps + 3) / 4;
  uint32_t P = C / E;
  if (P > kShrinkMaxParts) P = kShrinkMaxParts;
  if (P > n4) P = n4;
  return P < 2 ? PartPlan{0, 0} : PartPlan{E, P};
}

// Hidden steps [lo, hi) of part r of P (hi may pass h_steps: loads there
// read nothing): boundaries on multiples of 4 steps, so that they fall on
// pipeline-block boundaries of every kernel shape and depend only on the
// hidden size, P and r.
struct StepSpan {
  int32_t lo, hi;
};
constexpr StepSpan part_steps(uint32_t r, uint32_t P, uint32_t h_steps) {
  const uint32_t n4 = (h_steps + 3) / 4;
  return StepSpan{int32_t(4 * (r * n4 / P)), int32_t(4 * ((r + 1) * n4 / P))};
}

// Workspace layout: C 32-bit part counters (zero between calls), padded to
// 256 bytes, then C parts of kShrinkPartBytes.
constexpr int64_t shrink_workspace_counter_bytes(int64_t C) { return (4 * C + 255) / 256 * 256; }
constexpr int64_t shrink_workspace_bytes(int64_t C) {
  return shrink_workspace_counter_bytes(C) + C * int64_t(kShrinkPartBytes);
}

}  // namespace limits
}  // namespace sgmv
