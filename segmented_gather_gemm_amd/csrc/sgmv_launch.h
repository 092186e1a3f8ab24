// sgmv_launch.h -- interface between the host entry points (sgmv_api.cpp)
// and the gfx950 kernels (sgmv_kernels.hip).  Internal to libsgmv.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sgmv {

constexpr int kMaxSlices = 8;
constexpr int kThreads = 256;          // 4 wavefronts of 64 lanes
constexpr int kWaves = kThreads / 64;
constexpr int kWaveCols = 64;          // output columns one wavefront owns per unit
constexpr int kTileCols = kWaves * kWaveCols;  // columns per work unit (256)
constexpr int kTileRows = 16;          // rows per work unit (one MFMA column block)
constexpr int kColumnGroups = 8;       // one per XCD: the fast kernels' walk order
// Segment tables are ordered by adapter for batches in [min, max]: with many
// (short) segments, neighbours that share an adapter share weight tiles; the
// ordering costs O(batches^2 / threads) per workgroup.
constexpr int kSortMinBatches = 128;
constexpr int kSortMaxBatches = 512;
static_assert(kSortMaxBatches % kThreads == 0 && kSortMaxBatches <= 512,
              "segments per thread when ordering; 9-bit segment index in the sort key");

// Bits of SliceDesc::flags: 16-byte vector access is legal for ...
enum : int32_t {
  kVecX = 1,    // ... every 8-element block of an input row
  kVecW = 2,    // ... every 8-element block of a weight row
  kVecOut = 4,  // ... every 8-element column group of the output window
};

struct SliceDesc {
  const void* x;        // inputs (T, K), row stride x_stride elements
  const void* w;        // lora_b (L, N, K) contiguous
  int64_t x_stride;
  int64_t x_row_bytes;  // x_stride * sizeof(input element)
  int64_t n;            // slice_size
  int64_t offset;       // slice_offset
  int32_t tile_begin;   // first global column-tile index of this slice
  int32_t flags;
};

struct Params {
  void* out;
  const int64_t* start;
  const int64_t* lens;
  const int64_t* idx;
  int64_t out_stride;   // elements
  int64_t out_row_bytes;  // out_stride * sizeof(output element)
  int64_t T;            // rows of out (and of every inputs matrix)
  int32_t batches;
  int32_t L;            // lora_num
  int32_t K;            // rank
  int32_t num_slices;
  int32_t total_tiles;  // column tiles over all slices
  int32_t grid;         // workgroups launched
  int32_t band_tiles;   // row tiles per band of the fast kernels' walk
  int32_t chunk_units;  // fast kernels: units per chunk of the strided assignment
  int32_t sort_slots;   // order the segment table by adapter (batches <= kSortMaxBatches)
  int32_t per_token;    // segment b is row b alone (start and lens unused)
  int32_t gather;       // per-token table cut into gathered row tiles (fast kernels <..., true>)
  SliceDesc s[kMaxSlices];
};

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
  int64_t x_row_bytes;
  int64_t T;
  int32_t H;              // hidden size (< 2^26)
  int32_t batches;
  int32_t L;
  int32_t K;              // rank, the same for every slice
  int32_t num_slices;
  int32_t grid;
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
//    lora_A traffic per input row.
// Template shape: K16 = 16-row tiles of K per slice (1, 2, 4, 8, 16), NS =
// slices per launch (1..3), K16 * NS <= 16.
constexpr int kShrinkMaxSlicesPerLaunch = 3;
constexpr int kShrinkTokensSplitT = 64;

// Hidden steps (32 wide) per pipeline block.  Split-H: as many as keep about
// 64 registers of loads in flight per block.  Split-T: the block's lora_A
// tiles (tiles x steps KiB, two buffers) fit 64 KiB of LDS; the step count
// is 4 or 2 (even: each load covers two steps).
constexpr int shrink_block_steps_h(int xd, int tiles) {
  const int regs = 4 * ((xd == 2 ? 2 : 1) + tiles);
  return regs <= 8 ? 8 : regs <= 16 ? 4 : regs <= 32 ? 2 : 1;
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

// Kernel entries, by dtype codes (F16 = 0, BF16 = 1, F32 = 2), accumulate
// flag and, for the fast kernels, the number of 32-wide rank steps they hold
// in registers (rank <= 32 * steps; ks0: rank <= 16, one step, input tile not
// shared between waves) and whether row tiles gather per-token rows (the
// caller sets Params::gather to match).  nullptr: no such kernel.
//
// Fast kernels need rank % 8 == 0, every slice width % 8 == 0 and 16-byte
// aligned input rows, weight rows and output column groups; the generic
// kernel takes any shape, stride and alignment.
const void* fast_kernel_ks0(int xd, int wd, int od, bool add, bool gather);
const void* fast_kernel_ks1(int xd, int wd, int od, bool add, bool gather);
const void* fast_kernel_ks2(int xd, int wd, int od, bool add, bool gather);
const void* fast_kernel_ks4(int xd, int wd, int od, bool add, bool gather);
const void* fast_kernel_ks8(int xd, int wd, int od, bool add, bool gather);
const void* generic_kernel(int xd, int wd, int od, bool add);

}  // namespace sgmv
