// sgmv_fused_launch.h -- interface between the fused LoRA entry point
// (sgmv_fused_api.cpp) and its gfx950 kernels (sgmv_fused.h, instantiated
// in sgmv_fused_k*.hip).  Internal to libsgmv.
#pragma once

#include "sgmv_launch.h"
#include "sgmv_shrink_launch.h"

namespace sgmv {

// ---------------------------------------------------------------------------
// Fused LoRA delta: for each slice s, the LoRA-A projection of the inputs
// (the shrink, y_s = scale * x . A_s[a]^T, rounded to the 16-bit weight
// dtype and kept on chip) followed by the expand of y_s into the slice's
// output window (out[t][off_s + n] (+)= y_s[t] . B_s[a][n]).
// ---------------------------------------------------------------------------

constexpr int kFusedMaxSlices = kShrinkMaxSlicesPerLaunch;  // 3: QKV, gate/up
constexpr int kFusedTokens = kShrinkTokensSplitT;           // 64 tokens per unit

struct FusedSliceDesc {
  const void* a;        // lora_A (L, K, H) contiguous (field name as ShrinkSliceDesc)
  const void* w;        // lora_B (L, N, K) contiguous
  int64_t n;            // slice_size
  int64_t offset;       // slice_offset
  int32_t tile_begin;   // first global 256-column tile of this slice
  int32_t pad;
};

// Field names of the inputs and segment metadata match ShrinkParams (the
// segment-table builder and the split-T contraction take either).
struct FusedParams {
  const void* x;          // inputs (T, H), row stride x_row_bytes
  const int64_t* start;
  const int64_t* lens;
  const int64_t* idx;
  int64_t x_row_bytes;
  int64_t T;
  int32_t H;              // hidden size (< 2^26)
  int32_t batches;
  int32_t L;
  int32_t K;              // rank, the same for every slice
  int32_t num_slices;
  int32_t grid;
  int32_t cus;            // compute units of the device
  int32_t steps;          // 32-wide hidden steps per unit, whole turns of the ring
  int32_t sort_slots;
  int32_t per_token;      // always 0
  int32_t gather;         // always 0
  float scale;
  int32_t total_tiles;    // 256-column tiles over all slices
  int32_t item_target;    // split-H form: work items to aim for; a unit of U gets
                          // max(1, min(total_tiles, item_target / U)) column groups
  void* out;              // (T, H_out), row stride out_row_bytes
  int64_t out_row_bytes;
  FusedSliceDesc s[kFusedMaxSlices];
};

// Fused kernels by dtype codes (inputs, weights, output), accumulate flag
// and (k16, ns): k16 = 16-row k tiles per slice (1, 2, 4, 8), ns = slices
// (1..3), k16 * ns <= 16; nullptr if there is none.  Two forms: split_h
// (small batches: 16-row units, each in column groups sized from
// p.item_target; the split-H shrink's contraction) or split-T (64-row units; the split-T
// shrink's contraction).  They need K % 8 == 0,
// H % 8 == 0, slice widths % 8 == 0 and 16-byte aligned rows, weight stacks
// and output column windows.
const void* fused_kernel_k1(int xd, int wd, int od, bool add, int ns, bool split_h);
const void* fused_kernel_k2(int xd, int wd, int od, bool add, int ns, bool split_h);
const void* fused_kernel_k4(int xd, int wd, int od, bool add, int ns, bool split_h);
const void* fused_kernel_k8(int xd, int wd, int od, bool add, int ns, bool split_h);

}  // namespace sgmv
