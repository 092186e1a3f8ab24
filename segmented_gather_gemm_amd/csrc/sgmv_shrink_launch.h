// sgmv_shrink_launch.h -- interface between the shrink entry points
// (sgmv_shrink_api.cpp) and the gfx950 shrink kernels (sgmv_shrink_*.hip).
// Internal to libsgmv.
#pragma once

#include "sgmv_launch.h"

namespace sgmv {

// ---------------------------------------------------------------------------
// LoRA-A projection (shrink): y_s[t][k] = scale * sum_h x[t][h] * A_s[a][k][h]
// for the rows t of active segments, for every slice s (lora_A stack A_s
// (L, K, H) and output y_s (T, K)); the slices share the input.
// ---------------------------------------------------------------------------

struct ShrinkSliceDesc {
  const void* a;          // lora_A (L, K, H) contiguous
  void* out;              // (T, K), row stride out_row_bytes
  int64_t out_row_bytes;
};

// Field names of the segment metadata match Params (the segment-table
// builder takes either).
struct ShrinkParams {
  const void* x;          // inputs (T, H), row stride x_row_bytes
  const int64_t* start;
  const int64_t* lens;
  const int64_t* idx;
  void* ws;               // split-T parts workspace (limits::part_plan), or null
  int64_t x_row_bytes;
  int64_t T;
  int32_t H;              // hidden size (< 2^26)
  int32_t batches;
  int32_t L;
  int32_t K;              // rank, the same for every slice
  int32_t num_slices;
  int32_t grid;
  int32_t cus;            // compute units of the device
  int32_t steps;          // fast kernels: 32-wide hidden steps per wave (split-H) or per unit (split-T)
  int32_t sort_slots;
  int32_t per_token;
  int32_t gather;         // always 0 (no gathered row tiles here)
  float scale;
  ShrinkSliceDesc s[kMaxSlices];
};

// The fast shrink kernels come in two forms over the same contraction:
//  * split-H: a unit is 16 tokens; the four waves split the hidden steps and
//    add their partial sums through LDS.  Four times the units of split-T,
//    for small batches.
//  * split-T: a unit is 64 tokens, 16 per wave; every wave runs all hidden
//    steps and the lora_A rows of a block of steps are loaded once per
//    workgroup into LDS and read by all four waves -- a quarter of split-H's
//    lora_A traffic per input row.  With a workspace (ShrinkParams::ws),
//    batches of C < U <= 2 C or U <= C / 2 units run balanced
//    (limits::part_plan).
// Template shape: K16 = 16-row tiles of K per slice (1, 2, 4, 8, 16), NS =
// slices per launch (1..3), K16 * NS <= 16.
constexpr int kShrinkMaxSlicesPerLaunch = 3;
constexpr int kShrinkTokensSplitT = 64;

// Split-T (64-token units, lora_A shared through LDS) once the batch has at
// least this many 64-token units; split-H (16-token units) below, where it
// keeps more compute units busy.  The fused shrink-expand call takes the
// same form by the same rule, so that it reproduces the workspace-free
// shrink's sums.
#ifndef SGMV_SHRINK_SPLIT_T_MIN_UNITS
#define SGMV_SHRINK_SPLIT_T_MIN_UNITS 64
#endif
// Ranks up to 16 (one k tile per slice; lora_A is a small share of split-H's
// traffic): split-H stays ahead through 128 units of 64 tokens, i.e. two
// 16-token units per compute unit (measured, hidden 4096, 1-3 slices,
// workspace-balanced split-T: 66 units 1.06-1.31x, 128 units 1.01-1.19x in
// favour of split-H; 160-224 units 0.61-0.93x).
#ifndef SGMV_SHRINK_SPLIT_T_MIN_UNITS_NARROW
#define SGMV_SHRINK_SPLIT_T_MIN_UNITS_NARROW 129
#endif
// Units of 64 tokens from which a batch takes split-T, by 16-row k tiles per
// slice (a function of the rank alone, so that a multi-slice call takes its
// single calls' form).
constexpr int64_t shrink_split_t_min_units(int k16) {
  return k16 == 1 ? SGMV_SHRINK_SPLIT_T_MIN_UNITS_NARROW : SGMV_SHRINK_SPLIT_T_MIN_UNITS;
}

// Hidden steps (32 wide) per pipeline block.  Split-H: as many as keep about
// 64 registers of loads in flight per block.  Split-T: the block's lora_A
// tiles (tiles x steps KiB, two buffers) fit 64 KiB of LDS; the step count
// is 4 or 2 (even: each load covers two steps).
constexpr int shrink_block_steps_h(int xd, int tiles) {
  const int regs = 4 * ((xd == 2 ? 2 : 1) + tiles);
  const int steps = regs <= 8 ? 8 : regs <= 16 ? 4 : regs <= 32 ? 2 : 1;
  return tiles <= 8 && steps < 2 ? 2 : steps;  // coalesced loads (tiles <= 8) cover >= 2 steps
}
constexpr int shrink_block_steps_t(int tiles) {
  return tiles <= 4 ? 4 : 2;  // even: the loads cover two steps
}

// 16-byte loads one wave issues per block, and the number of blocks in
// flight (a ring of stages in registers, even, 2..8): as many as fit about
// 128 registers, so that a wave keeps up to 32 KiB of loads outstanding.
constexpr int shrink_block_loads_h(int xd, int tiles) {
  return shrink_block_steps_h(xd, tiles) * ((xd == 2 ? 2 : 1) + tiles);
}
constexpr int shrink_block_loads_t(int xd, int k16, int ns) {
  return shrink_block_steps_t(k16 * ns) * (xd == 2 ? 2 : 1) +
         ns * (k16 * shrink_block_steps_t(k16 * ns) / 4);
}
constexpr int shrink_ring(int block_loads) {
  const int d = (32 / block_loads) & ~1;
  return d < 2 ? 2 : d > 8 ? 8 : d;
}

// Shrink kernels by dtype codes and (k16, ns); nullptr if there is none.
// Fast kernels need K % 8 == 0, H % 8 == 0, 16-byte aligned rows and
// H < 2^26; the generic one takes any shape, stride and alignment.
const void* shrink_kernel_k1(int xd, int wd, int od, int ns, bool split_t);
const void* shrink_kernel_k2(int xd, int wd, int od, int ns, bool split_t);
const void* shrink_kernel_k4(int xd, int wd, int od, int ns, bool split_t);
const void* shrink_kernel_k8(int xd, int wd, int od, int ns, bool split_t);
const void* shrink_kernel_k16(int xd, int wd, int od, int ns, bool split_t);
const void* shrink_generic_kernel(int xd, int wd, int od);

}  // namespace sgmv
