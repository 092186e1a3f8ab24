// sgmv_launch.h -- interface between the host entry points (sgmv_api.cpp)
// and the gfx950 expand kernels (sgmv_device.h, instantiated in
// sgmv_fast_ks*.hip and sgmv_generic.hip).  Internal to libsgmv.
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
// Segment tables are ordered by adapter for batches in [min, max], and for
// any batch count up to max when the call holds at least kSortMinUnits work
// units and one adapter's weights (all slices) are at least
// kSortMinAdapterBytes: segments that share an adapter are then neighbours
// in the walk and share its weight tiles (from registers or L2) instead of
// fetching them again from memory.  The ordering costs O(batches^2 /
// threads) per workgroup (a few tenths of a microsecond) and changes the
// walk's balance; measured on MI355X it pays where weights are a large part
// of the traffic (14336-wide slice at rank 64: 108.9 -> 105.8 us) and not
// where they are small (fused QKV at rank 32: 55.1 -> 56.1 us).
constexpr int kSortMinBatches = 128;
constexpr int kSortMaxBatches = 512;
#ifndef SGMV_SORT_MIN_UNITS
#define SGMV_SORT_MIN_UNITS 8192
#endif
constexpr int64_t kSortMinUnits = SGMV_SORT_MIN_UNITS;
constexpr int64_t kSortMinAdapterBytes = int64_t(1) << 20;
// Per-token calls gather each adapter's tokens into row tiles for up to this
// many tokens (every per-token call the ABI accepts, SGMV_MAX_BATCHES) and
// adapters (the gathered table: tokens + 2 adapters + 1 LDS words; each
// unit's decode scans the tokens once).  Measured on q_proj shapes with 32
// adapters, gathering beats one-token tiles 3-3.6x from 1024 to 4000 tokens.
constexpr int kGatherMaxTokens = 4000;
constexpr int kGatherMaxAdapters = 1024;
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
  int32_t cus;          // compute units of the device
  int32_t band_tiles;   // row tiles per band of the fast kernels' walk
  int32_t chunk_units;  // fast kernels: units per chunk of the strided assignment
  int32_t sort_slots;   // order the segment table by adapter (batches <= kSortMaxBatches)
  int32_t per_token;    // segment b is row b alone (start and lens unused)
  int32_t gather;       // gathered per-token row tiles (fast kernels <..., true>)
  SliceDesc s[kMaxSlices];
};

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
// Vector-ALU form for rank <= 32 (sgmv_valu.hip), same shape requirements as
// the fast kernels, no gathered tiles; the host takes it only in builds with
// SGMV_EXPAND_VALU defined (a measurement of the matrix-core choice).
const void* valu_kernel(int xd, int wd, int od, bool add);

}  // namespace sgmv
