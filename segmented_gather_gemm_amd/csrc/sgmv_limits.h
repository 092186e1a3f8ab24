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

// Balanced split-T shrink (calls that bring a workspace; C compute units,
// C % 8 == 0; a unit alone takes ~40 us at hidden 4096 whatever else runs
// beside it, so the time is set by the compute units with the most work):
//  * C < U <= 2 C units: some compute units would run two units where the
//    others run one.  Workgroups 0..C-1 take one unit each (W = C whole
//    units, unit_span over them) and the E = U - C other units are cut into
//    P = min(C / E, kShrinkMaxParts, ceil(h_steps / 4)) parts over the
//    hidden steps;
//  * U <= C / 2: most compute units would idle while each unit takes a
//    unit's time.  Every unit is cut into P = min(C / U, ...) parts (W = 0,
//    E = U).
// The E P parts, in unit order, go to workgroups W, W + 1, ... XCD by XCD
// (part_item): XCD x takes the x-th of 8 contiguous shares (sizes differ by
// at most one, at most C / 8), so that neighbouring units -- one segment's,
// or one adapter's in an adapter-ordered table -- and so their lora_A rows
// stay on one XCD's L2 (a unit's parts straddle two XCDs only at a share's
// end; dealing consecutive parts to consecutive XCDs instead measured
// slower on batches where neighbouring units share an adapter: 128 units
// of 64 tokens, 34.0 against 39.8 us).  Parts write fp32 partial sums to
// the workspace; the last part of a unit to finish adds them in part order
// and stores the result.  plan.P == 0: the call does not qualify
// (workspace-free launch, C / 2 < U <= C or U > 2 C, a grid below W + C, or
// P < 2: with more than 1.5 C units whole overflow units on workgroups C..
// measured 4-5% slower than unit_span's XCD-major fill) and the units are
// split by unit_span.
#ifndef SGMV_SHRINK_MAX_PARTS
#define SGMV_SHRINK_MAX_PARTS 4
#endif
constexpr uint32_t kShrinkMaxParts = SGMV_SHRINK_MAX_PARTS;
// Workspace bytes of one part's partial sums: 64 tokens x 256 rows (16 k
// tiles, the most one launch takes) of fp32.
constexpr uint32_t kShrinkPartBytes = 64u * 256u * 4u;

struct PartPlan {
  uint32_t W, E, P;  // whole units (on workgroups 0..W-1), overflow units, parts per overflow unit
};
constexpr PartPlan part_plan(uint32_t U, uint32_t C, uint32_t G, uint32_t h_steps) {
  if (C < 8 || (C & 7) != 0 || U == 0 || U > 2 * C || h_steps == 0) return PartPlan{0, 0, 0};
  const uint32_t W = U > C ? C : 0, E = U - W, n4 = (h_steps + 3) / 4;
  uint32_t P = C / E;
  if (P > kShrinkMaxParts) P = kShrinkMaxParts;
  if (P > n4) P = n4;
  if (P < 2 || G < W + C) return PartPlan{0, 0, 0};
  return PartPlan{W, E, P};
}

// The part workgroup `bid` (>= plan.W) runs: part `part` of unit `unit`,
// with workspace slot (unit - W) P + part, or nothing (valid false).  bid
// and bid - W have the same XCD (W % 8 == 0); XCD x's share of the parts
// (slot order) is [x E P/8, (x + 1) E P/8), taken by its workgroups in
// order of (bid - W) / 8.
struct PartItem {
  uint32_t unit, part;
  bool valid;
};
constexpr PartItem part_item(const PartPlan& pl, uint32_t bid) {
  const uint32_t k = bid - pl.W, x = k & 7, j = k >> 3, I = pl.E * pl.P;
  const uint32_t share = I >> 3, extra = I & 7;
  const uint32_t base = x * share + (x < extra ? x : extra);
  const uint32_t n = share + (x < extra ? 1u : 0u);
  if (j >= n) return PartItem{0, 0, false};
  const uint32_t slot = base + j;
  return PartItem{pl.W + slot / pl.P, slot % pl.P, true};
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
